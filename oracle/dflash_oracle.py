"""CPU oracle for the DFlash draft-proposal path.  TEST INFRASTRUCTURE ONLY.

Only tests/, __graft_entry__.smoke() and bench.py's cpu_baseline leg may import or call this
module. The product (the HIP library and its Python binding) never does, and shares no code,
table or constant generator with it.

This is a plain, slow, fp64 numpy implementation of what the method computes, written from
three web pages:

  [N] "DFlash Speculative Decoding in the vLLM Neuron Framework" (AWS Neuron design doc)
  [V] "[Feat][Spec Decode] DFlash" (vLLM pull request #36847: tests and review)
  [Q] "Dflash: Block Diffusion Speculative Decoding" (Qualcomm efficient-transformers PR #995)

The pages fix neither the precision nor several details of the layer. Where they are silent
the docstrings below say "reading" and state the reading taken.

Storage rounding (reading: the pages fix no precision).  Weights and the KV cache are held in
the drafter's storage type (bf16 or fp32); the block's own q, k and v, which enter attention
alongside cached keys and values, are rounded to it as well. Every other activation, including
every GEMM input, the residual stream, norms, softmax and logits, is kept unrounded here (fp64).
That too is a reading the pages do not fix: an implementation may keep those activations in
fp32 and may feed a bf16 matrix unit an approximation of them (for instance the pair
hi = bf16(f), lo = bf16(f - hi), which keeps 17 significant bits of f); parity tolerances then
absorb the difference. Rounding every GEMM input to bf16 instead would make two correct
implementations drift apart by about one bf16 unit per element after a few layers, since each
rounding disagreement is spread by the next dense product into the following rounding point.
The oracle computes in fp64 and rounds at exactly the points above (`rho`). mode="exact" turns
all rounding off (a precision diagnostic, and what the transformers-based pins compare against).

Parity unpinned: the bf16-mode storage rounding points. They are a reading (the pages fix no
precision), and no pin fixes where rounding happens; the pins below run in mode="exact" or
check the rounding function itself.

Array conventions: dense weights are row-major [out, in] (y = W x, the F.linear convention).
Each KV cache is a list over layers of float32 arrays [num_pages, page_size, n_kv_heads,
head_dim]; a flat slot s is page s // page_size, offset s % page_size.

Pins: every function here is checked by tests/test_oracle_*.py against things other than
itself (transformers' Qwen3 layers, torch's bf16 cast and SDPA, a complex-number RoPE,
brute-force greedy decoding, the worked example printed in [V], hand-worked slot mappings).
"""
from __future__ import annotations

import numpy as np

# --------------------------------------------------------------------------------------------
# Storage rounding
# --------------------------------------------------------------------------------------------
_BF16_MAX = float.fromhex("0x1.fep127")  # largest finite bfloat16
_BF16_OVERFLOW = float.fromhex("0x1.ffp127")  # halfway to 2^128: RNE overflows from here on


def round_bf16(x) -> np.ndarray:
    """Round fp64 values to the nearest bfloat16 value, ties to even.

    bfloat16 keeps fp32's exponent range with 8 significant bits: the spacing of the grid in
    the binade [2^(e-1), 2^e) is 2^(e-8). Below the smallest normal (2^-126) the spacing stays
    2^-133 (subnormals)."""
    x = np.asarray(x, dtype=np.float64)
    _, e = np.frexp(x)  # x = m 2^e with 0.5 <= |m| < 1
    q = np.maximum(e, -125) - 8  # log2 of the grid spacing
    r = np.ldexp(np.rint(np.ldexp(x, -q)), q)  # np.rint rounds half to even
    r = np.where(np.abs(x) >= _BF16_OVERFLOW, np.copysign(np.inf, x), r)
    return np.where(np.isfinite(x), r, x)


def round_f32(x) -> np.ndarray:
    return np.asarray(x, dtype=np.float64).astype(np.float32).astype(np.float64)


def storage_rounding(mode: str):
    """rho: 'bf16' and 'f32' round to that storage type; 'exact' is the identity."""
    if mode == "bf16":
        return round_bf16
    if mode == "f32":
        return round_f32
    if mode == "exact":
        return lambda a: np.asarray(a, dtype=np.float64)
    raise ValueError(mode)


def f64(a) -> np.ndarray:
    return np.asarray(a, dtype=np.float64)


# --------------------------------------------------------------------------------------------
# Layer pieces
# --------------------------------------------------------------------------------------------
def rms_norm(x, w, eps: float) -> np.ndarray:
    """RMSNorm over the last axis: x / sqrt(mean(x^2) + eps) * w.

    Reading: hidden_norm, the pre-norms, q/k norms and the final norm are all this Qwen3
    RMSNorm with a learned weight ([N] "Context KV Injection" step 1 names hidden_norm; the
    layer is "a standard Qwen3 decoder layer ... with pre-norms", [N] "DFlash Draft Model
    Architecture")."""
    x = f64(x)
    ms = np.mean(x * x, axis=-1, keepdims=True)
    return x / np.sqrt(ms + eps) * f64(w)


def rope_inv_freq(head_dim: int, theta: float) -> np.ndarray:
    i = np.arange(head_dim // 2, dtype=np.float64)
    return float(theta) ** (-2.0 * i / head_dim)


def apply_rope(x, pos, theta: float) -> np.ndarray:
    """Rotary position embedding, rotate-half pairing (element i pairs with i + D/2).

    x: [..., D]; pos: integer positions broadcastable to x.shape[:-1]. Positions are absolute
    ([Q] commit message on the model-level rotary table: it is gathered by absolute position).
    Reading: Qwen3's pairing and inv_freq_i = theta^(-2i/D), no scaling."""
    x = f64(x)
    D = x.shape[-1]
    half = D // 2
    ang = f64(pos)[..., None] * rope_inv_freq(D, theta)
    c, s = np.cos(ang), np.sin(ang)
    x1, x2 = x[..., :half], x[..., half:]
    return np.concatenate([x1 * c - x2 * s, x2 * c + x1 * s], axis=-1)


def silu(x) -> np.ndarray:
    x = f64(x)
    return x / (1.0 + np.exp(-x))


def attention(q, k, v) -> np.ndarray:
    """softmax(q k^T / sqrt(D)) v for one head.  q [Tq, D], k/v [Tk, D] -> [Tq, D].

    No mask: every query sees every key ([V] test of the first pass asserts causal is False;
    [N] "What is DFlash": each query attends to the injected context and the rest of the
    block)."""
    q, k, v = f64(q), f64(k), f64(v)
    s = q @ k.T / np.sqrt(q.shape[-1])
    s = s - s.max(axis=-1, keepdims=True)
    p = np.exp(s)
    p /= p.sum(axis=-1, keepdims=True)
    return p @ v


def paged_slots(block_table, req_ids, positions, page_size: int) -> np.ndarray:
    """Flat cache slot of (request, absolute position) ([N] "Paged KV Integration"):
    the page number is pos // page_size clamped to the table width, the physical page comes
    from the request's block-table row, and the slot is page * page_size + pos % page_size."""
    bt = np.asarray(block_table, dtype=np.int64)
    pos = np.asarray(positions, dtype=np.int64)
    bn = np.minimum(pos // page_size, bt.shape[1] - 1)
    return bt[np.asarray(req_ids, dtype=np.int64), bn] * page_size + pos % page_size


# --------------------------------------------------------------------------------------------
# KV injection ([N] "Context KV Injection (Precompute)")
# --------------------------------------------------------------------------------------------
def inject_context_kv(spec, W, k_cache, v_cache, aux, positions, slot_mapping, mode: str):
    """Write the context rows' K/V into every draft layer's paged cache, in place.

    aux: list of n_aux arrays [N, target_hidden] in ascending target-layer order. Their
    concatenation along features is the [N, n_aux * target_hidden] input ([N] "Target
    Auxiliary Hidden State Extraction"). Then ctx = hidden_norm(fc(concat)) (step 1). Each
    layer's K = k_norm then RoPE at the row's position, and V = the plain projection, go to
    slot_mapping[r] (steps 2 and 3). Rows with a negative slot are padding and are skipped.

    Reading: context K/V see hidden_norm only, not the layer's input norm (step 2 applies
    the fused K/V projection to ctx directly). Fusing the layers' K/V weights into one matrix
    is a re-association of the same product, so per-layer projections are used here.

    Returns {"y": fc output, "ctx": hidden_norm output} for the kept rows."""
    rho = storage_rounding(mode)
    slot = np.asarray(slot_mapping, dtype=np.int64)
    keep = np.nonzero(slot >= 0)[0]
    pos = np.asarray(positions, dtype=np.int64)[keep]
    x = np.concatenate([f64(a)[keep] for a in aux], axis=1)
    y = x @ f64(W["fc"]).T
    ctx = rms_norm(y, W["hidden_norm"], spec.rms_eps)  # a GEMM input: kept exact
    P = k_cache[0].shape[1]
    page, off = slot[keep] // P, slot[keep] % P
    KVH, D = spec.n_kv_heads, spec.head_dim
    for l in range(spec.n_layers):
        p = f"layers.{l}."
        k = (ctx @ f64(W[p + "wk"]).T).reshape(-1, KVH, D)
        v = (ctx @ f64(W[p + "wv"]).T).reshape(-1, KVH, D)
        k = rho(apply_rope(rms_norm(k, W[p + "k_norm"], spec.rms_eps), pos[:, None], spec.rope_theta))
        k_cache[l][page, off] = k
        v_cache[l][page, off] = rho(v)
    return {"y": y, "ctx": ctx, "rows": keep}


# --------------------------------------------------------------------------------------------
# Block proposal
# --------------------------------------------------------------------------------------------
def build_query_block(bonus, seq_lens, block_size: int, mask_token_id: int):
    """The [bonus, mask, ..., mask] query block of every request ([N] "Draft Block
    Construction"; [V] test of the first pass for DFlash).

    Returns the flattened ids, positions seq_len + [0 .. block_size-1], the indices of the
    kept (mask) rows, and query_start_loc."""
    bonus = np.asarray(bonus, dtype=np.int64)
    c = np.asarray(seq_lens, dtype=np.int64)
    B = bonus.shape[0]
    ids = np.full((B, block_size), mask_token_id, dtype=np.int64)
    ids[:, 0] = bonus
    positions = c[:, None] + np.arange(block_size)[None, :]
    keep = (np.arange(B)[:, None] * block_size + np.arange(1, block_size)[None, :]).reshape(-1)
    qsl = np.arange(B + 1, dtype=np.int64) * block_size
    return ids.reshape(-1), positions.reshape(-1), keep, qsl


def _lm_head_argmax(f, U, chunk: int = 8192):
    """Greedy token of every row of f: the lowest index among the maximal logits of U f.

    Logits stay fp64 and are never rounded (reading: rounding them would create ties).
    Also returns the gap between the largest and second-largest logit."""
    f = f64(f)
    V = U.shape[0]
    z = np.empty((f.shape[0], V), dtype=np.float64)
    for c0 in range(0, V, chunk):
        z[:, c0:c0 + chunk] = f @ f64(U[c0:c0 + chunk]).T
    tok = np.argmax(z, axis=1)  # first index of the maximum
    top2 = np.partition(z, V - 2, axis=1)[:, V - 2:]
    return tok, top2[:, 1] - top2[:, 0], z


def propose_block(spec, W, k_cache, v_cache, block_table, bonus, seq_lens, mode: str,
                  page_size: int | None = None, return_logits: bool = False):
    """One non-causal block forward of the drafter and greedy drafting ([N] "DFlash Draft
    Model Architecture", forward()).

    For every request b the block [bonus_b, mask x K] sits at positions c_b + j, c_b =
    seq_lens[b] being the number of injected context tokens. It is embedded with the target
    embedding, then runs n_layers Qwen3 decoder layers. In each, every block query attends,
    without a mask, to the c_b context keys read from the paged cache and to all block_size
    block keys. The block's own K/V are not written to the cache (reading). Rows 1..K are
    kept, passed through the final norm (reading) and the target LM head, and argmax gives
    the drafts.

    Returns dict(draft_token_ids [B, bs], drafts_only [B, K], hidden [B*K, H] (final-norm
    output), gap [B, K] top-2 logit gap, and optionally logits)."""
    rho = storage_rounding(mode)
    H, QH, KVH, D = spec.hidden, spec.n_q_heads, spec.n_kv_heads, spec.head_dim
    G = QH // KVH
    bs, K, eps = spec.block_size, spec.block_size - 1, spec.rms_eps
    P = page_size if page_size is not None else k_cache[0].shape[1]
    bonus = np.asarray(bonus, dtype=np.int64)
    c = np.asarray(seq_lens, dtype=np.int64)
    B = bonus.shape[0]
    ids, pos, keep, _ = build_query_block(bonus, c, bs, spec.mask_token_id)

    x = f64(np.asarray(W["embed"])[ids])  # residual stream [B*bs, H], never rounded
    for l in range(spec.n_layers):
        p = f"layers.{l}."
        h = rms_norm(x, W[p + "in_norm"], eps)
        q = (h @ f64(W[p + "wq"]).T).reshape(-1, QH, D)
        k = (h @ f64(W[p + "wk"]).T).reshape(-1, KVH, D)
        v = (h @ f64(W[p + "wv"]).T).reshape(-1, KVH, D)
        q = rho(apply_rope(rms_norm(q, W[p + "q_norm"], eps), pos[:, None], spec.rope_theta))
        k = rho(apply_rope(rms_norm(k, W[p + "k_norm"], eps), pos[:, None], spec.rope_theta))
        v = rho(v)
        o = np.empty((B * bs, QH, D), dtype=np.float64)
        for b in range(B):
            rows = slice(b * bs, (b + 1) * bs)
            t = np.arange(c[b])
            slots = paged_slots(block_table, np.full_like(t, b), t, P)
            kc = f64(k_cache[l][slots // P, slots % P])  # [c_b, KVH, D]
            vc = f64(v_cache[l][slots // P, slots % P])
            keys = np.concatenate([kc, k[rows]], axis=0)
            vals = np.concatenate([vc, v[rows]], axis=0)
            for hq in range(QH):
                g = hq // G  # reading: q head h uses kv head h // G
                o[rows, hq] = attention(q[rows, hq], keys[:, g], vals[:, g])
        x = x + o.reshape(B * bs, QH * D) @ f64(W[p + "wo"]).T
        h2 = rms_norm(x, W[p + "post_norm"], eps)
        gate = h2 @ f64(W[p + "w_gate"]).T
        up = h2 @ f64(W[p + "w_up"]).T
        x = x + (silu(gate) * up) @ f64(W[p + "w_down"]).T

    f = rms_norm(x[keep], W["final_norm"], eps)
    tok, gap, z = _lm_head_argmax(f, W["lm_head"])
    drafts = tok.reshape(B, K).astype(np.int32)
    out = {"draft_token_ids": np.concatenate([bonus[:, None].astype(np.int32), drafts], axis=1),
           "drafts_only": drafts, "hidden": f, "gap": gap.reshape(B, K)}
    if return_logits:
        out["logits"] = z
    return out


# --------------------------------------------------------------------------------------------
# Greedy verification
# --------------------------------------------------------------------------------------------
def greedy_verify(drafts, target):
    """Greedy verification of K drafts against the target's K+1 argmax tokens.

    The target's token i is its greedy choice after the context plus drafts[:i]. The accepted
    length a = (length of the longest prefix where drafts[i] == target[i]) + 1. The emitted
    tokens are target[:a]; later entries are -1, the rejected marker of the greedy rejection
    sampler ([N] "Async Rejection and Position Correction"). The next bonus is target[a-1].
    Output equals standard greedy decoding ([Q] description: verification by the frozen
    target)."""
    drafts = np.asarray(drafts, dtype=np.int64)
    target = np.asarray(target, dtype=np.int64)
    B, K = drafts.shape
    a = np.empty(B, dtype=np.int32)
    out = np.full((B, K + 1), -1, dtype=np.int32)
    nb = np.empty(B, dtype=np.int32)
    for b in range(B):
        n = 0
        while n < K and drafts[b, n] == target[b, n]:
            n += 1
        a[b] = n + 1
        out[b, :n + 1] = target[b, :n + 1]
        nb[b] = target[b, n]
    return a, out, nb


def acceptance_metrics(accepted_len, num_drafts_per_block: int):
    """The spec-decode counters and the two derived metrics of [V]'s acceptance tests:
    rate = accepted / draft tokens, length = 1 + accepted / drafts."""
    a = np.asarray(accepted_len, dtype=np.int64)
    num_drafts = int(a.size)
    num_draft_tokens = num_drafts * num_drafts_per_block
    num_accepted = int((a - 1).sum())
    rate = num_accepted / num_draft_tokens if num_draft_tokens else float("nan")
    length = 1 + num_accepted / num_drafts if num_drafts else 1.0
    return {"num_drafts": num_drafts, "num_draft_tokens": num_draft_tokens,
            "num_accepted_tokens": num_accepted, "acceptance_rate": rate,
            "acceptance_length": length}


# --------------------------------------------------------------------------------------------
# Proposal-input preparation ([N] "Async Rejection and Position Correction", "Paged KV
# Integration", "Draft Block Construction")
# --------------------------------------------------------------------------------------------
def prepare_proposal_inputs(prev_out, vocab: int, opt_seq_lens, row_req, opt_positions, block_table,
                            page_size: int):
    """Corrects an optimistically scheduled step once the previous verification is known.

    The scheduler prepared the step as if all K_prev drafts of the previous step had been
    accepted. For each request b the previous rejection-sampler output prev_out[b] (K_prev + 1
    entries: emitted tokens, -1 for rejected ones) gives
      valid_b    = number of entries that are not -1 and lie below the vocabulary size,
      rejected_b = (1 + K_prev) - valid_b,
    and the step is corrected by removing the rejected positions:
      seq_lens[b]   = opt_seq_lens[b] - rejected_b            (post-verification length)
      positions[r]  = opt_positions[r] - rejected_{row_req[r]} (context rows to inject)
      slots[r]      = paged slot of (row_req[r], positions[r])
      bonus[b]      = the last valid entry of prev_out[b] (the block's slot-0 token).
    A request with no valid entry keeps bonus 0, and a corrected position below 0 gets slot -1,
    which injection skips (readings: neither arises from a consistent schedule, the greedy
    rejection always emits at least one token)."""
    prev = np.asarray(prev_out, dtype=np.int64)
    B, K1 = prev.shape
    ok = (prev != -1) & (prev >= 0) & (prev < vocab)
    valid = ok.sum(axis=1)
    rejected = K1 - valid
    seq_lens = np.asarray(opt_seq_lens, dtype=np.int64) - rejected
    req = np.asarray(row_req, dtype=np.int64)
    positions = np.asarray(opt_positions, dtype=np.int64) - rejected[req]
    slots = np.where(positions >= 0, paged_slots(block_table, req, np.maximum(positions, 0), page_size), -1)
    bonus = np.zeros(B, dtype=np.int64)
    for b in range(B):
        idx = np.nonzero(ok[b])[0]
        if idx.size:
            bonus[b] = prev[b, idx[-1]]
    return {"seq_lens": seq_lens.astype(np.int32), "positions": positions.astype(np.int32),
            "slot_mapping": slots.astype(np.int64), "bonus": bonus.astype(np.int32),
            "num_rejected": rejected.astype(np.int32)}
