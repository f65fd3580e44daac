"""ctypes binding of libdflash (include/dflash.h): argument marshalling only.

Every step of the drafting path runs in the library's HIP kernels. PyTorch supplies device
memory and the current stream and nothing else. There is no fallback: if the library is
missing, `lib()` raises.

Names follow the C ABI: inject_context_kv, propose_block, greedy_verify, workspace_bytes,
build_rope_table, build_fused_kv_weight. `Drafter` bundles a drafter's device weights with the
ctypes structs that point at them.
"""
from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libdflash.so")

DFLASH_F32, DFLASH_BF16 = 0, 1
DFLASH_OP_INJECT, DFLASH_OP_PROPOSE = 0, 1

_vp = ctypes.c_void_p
_i32 = ctypes.c_int32


class Config(ctypes.Structure):
    _fields_ = [(n, _i32) for n in ("hidden", "n_layers", "n_q_heads", "n_kv_heads", "head_dim",
                                     "intermediate", "vocab", "n_aux", "target_hidden", "block_size",
                                     "mask_token_id")] + [("rms_eps", ctypes.c_float), ("dtype", _i32)]


_PER_LAYER = ("in_norm", "wq", "wk", "wv", "q_norm", "k_norm", "wo", "post_norm", "w_gate", "w_up", "w_down")


class Weights(ctypes.Structure):
    _fields_ = ([(n, _vp) for n in ("fc", "hidden_norm", "embed", "lm_head", "final_norm", "kv_fused")]
                + [(n, ctypes.POINTER(_vp)) for n in _PER_LAYER]
                + [("rope_cos", _vp), ("rope_sin", _vp), ("rope_max_pos", _i32)])


class KvCache(ctypes.Structure):
    _fields_ = [("k", ctypes.POINTER(_vp)), ("v", ctypes.POINTER(_vp)), ("num_pages", _i32),
                ("page_size", _i32), ("block_table", _vp), ("max_blocks_per_seq", _i32)]


class DFlashError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(message)
        self.status = status


_LIB = None


def lib() -> ctypes.CDLL:
    """The loaded library (raises if it has not been built)."""
    global _LIB
    if _LIB is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with __graft_entry__.build()")
        L = ctypes.CDLL(LIB_PATH)
        P = ctypes.POINTER
        L.dflash_build_rope_table.argtypes = [_i32, ctypes.c_double, _i32, _vp, _vp, _vp]
        L.dflash_build_fused_kv_weight.argtypes = [P(Config), P(Weights), _vp, _vp]
        L.dflash_workspace_bytes.argtypes = [P(Config), _i32, _i32, _i32]
        L.dflash_workspace_bytes.restype = ctypes.c_size_t
        L.dflash_inject_context_kv.argtypes = [P(Config), P(Weights), P(KvCache), P(_vp), ctypes.c_int64, _i32,
                                               _vp, _vp, _vp, ctypes.c_size_t, _vp]
        L.dflash_propose_block.argtypes = [P(Config), P(Weights), P(KvCache), _i32, _vp, _vp, _i32, _vp, _vp, _vp,
                                           _vp, ctypes.c_size_t, _vp]
        L.dflash_propose_block_after.argtypes = [P(Config), P(Weights), P(KvCache), _i32, _vp, _vp, _i32, _vp, _vp,
                                                 _vp, _vp, ctypes.c_size_t, _vp, _vp]
        L.dflash_propose_block_noalloc.argtypes = [P(Config), P(Weights), P(KvCache), _i32, _vp, _vp, _i32, _vp, _vp,
                                                   _vp, _vp]
        L.dflash_greedy_verify.argtypes = [_i32, _i32, _vp, _vp, _vp, _vp, _vp, _vp]
        L.dflash_greedy_verify_stats.argtypes = [_i32, _i32, _vp, _vp, _vp, _vp, _vp, _vp, _vp]
        L.dflash_prepare_proposal_inputs.argtypes = [_i32, _i32, _vp, _i32, _vp, _i32, _vp, _vp, _vp, _i32, _i32,
                                                     _vp, _vp, _vp, _vp, _vp]
        for fn in ("dflash_build_rope_table", "dflash_build_fused_kv_weight", "dflash_inject_context_kv",
                   "dflash_propose_block", "dflash_propose_block_after", "dflash_propose_block_noalloc",
                   "dflash_greedy_verify",
                   "dflash_greedy_verify_stats", "dflash_prepare_proposal_inputs"):
            getattr(L, fn).restype = _i32
        L.dflash_profile_enable.argtypes = [_i32]
        L.dflash_profile_enable.restype = _i32
        L.dflash_profile_collect.restype = _i32
        L.dflash_profile_filter.argtypes = [ctypes.c_char_p]
        L.dflash_profile_filter.restype = _i32
        L.dflash_profile_count.restype = _i32
        L.dflash_profile_entry.argtypes = [_i32, ctypes.POINTER(ctypes.c_char_p), ctypes.POINTER(ctypes.c_int64),
                                           ctypes.POINTER(ctypes.c_double)]
        L.dflash_profile_entry.restype = _i32
        L.dflash_status_string.argtypes = [_i32]
        L.dflash_status_string.restype = ctypes.c_char_p
        L.dflash_last_error.restype = ctypes.c_char_p
        _LIB = L
    return _LIB


def _check(status: int) -> None:
    if status != 0:
        L = lib()
        raise DFlashError(status, f"{L.dflash_status_string(status).decode()}: {L.dflash_last_error().decode()}")


def _ptr(t) -> int | None:
    return None if t is None else t.data_ptr()


def _stream(stream) -> int:
    s = stream if stream is not None else torch.cuda.current_stream()
    return s.cuda_stream


def make_config(spec) -> Config:
    """ctypes config from any object with the DrafterSpec fields."""
    return Config(spec.hidden, spec.n_layers, spec.n_q_heads, spec.n_kv_heads, spec.head_dim, spec.intermediate,
                  spec.vocab, spec.n_aux, spec.target_hidden, spec.block_size, spec.mask_token_id, spec.rms_eps,
                  DFLASH_BF16 if spec.dtype == "bf16" else DFLASH_F32)


def storage_dtype(spec) -> torch.dtype:
    return torch.bfloat16 if spec.dtype == "bf16" else torch.float32


# ----------------------------------------------------------------------------------------
# Raw entry points
# ----------------------------------------------------------------------------------------
def build_rope_table(head_dim: int, theta: float, max_pos: int, cos_out, sin_out, stream=None) -> None:
    _check(lib().dflash_build_rope_table(head_dim, theta, max_pos, _ptr(cos_out), _ptr(sin_out), _stream(stream)))


def build_fused_kv_weight(cfg: Config, w: Weights, out, stream=None) -> None:
    _check(lib().dflash_build_fused_kv_weight(ctypes.byref(cfg), ctypes.byref(w), _ptr(out), _stream(stream)))


def workspace_bytes(cfg: Config, op: int, max_rows_or_batch: int, max_context: int = 0) -> int:
    return int(lib().dflash_workspace_bytes(ctypes.byref(cfg), op, max_rows_or_batch, max_context))


def inject_context_kv(cfg, w, cache, aux, aux_row_stride, n_rows, positions, slot_mapping, workspace,
                      stream=None) -> None:
    arr = (_vp * len(aux))(*[_ptr(a) for a in aux])
    _check(lib().dflash_inject_context_kv(ctypes.byref(cfg), ctypes.byref(w), ctypes.byref(cache), arr,
                                          aux_row_stride, n_rows, _ptr(positions), _ptr(slot_mapping),
                                          _ptr(workspace), workspace.numel() * workspace.element_size(),
                                          _stream(stream)))


def propose_block(cfg, w, cache, batch, bonus_tokens, seq_lens, max_context, draft_token_ids, drafts_only,
                  hidden_out, workspace, stream=None) -> None:
    _check(lib().dflash_propose_block(ctypes.byref(cfg), ctypes.byref(w), ctypes.byref(cache), batch,
                                      _ptr(bonus_tokens), _ptr(seq_lens), max_context, _ptr(draft_token_ids),
                                      _ptr(drafts_only), _ptr(hidden_out), _ptr(workspace),
                                      workspace.numel() * workspace.element_size(), _stream(stream)))


def propose_block_after(cfg, w, cache, batch, bonus_tokens, seq_lens, max_context, draft_token_ids, drafts_only,
                        hidden_out, workspace, cache_ready=None, stream=None) -> None:
    """`cache_ready`: a torch.cuda.Event recorded after the step's injection (or None)."""
    ev = cache_ready.cuda_event if cache_ready is not None else None
    _check(lib().dflash_propose_block_after(ctypes.byref(cfg), ctypes.byref(w), ctypes.byref(cache), batch,
                                            _ptr(bonus_tokens), _ptr(seq_lens), max_context, _ptr(draft_token_ids),
                                            _ptr(drafts_only), _ptr(hidden_out), _ptr(workspace),
                                            workspace.numel() * workspace.element_size(), ev, _stream(stream)))


def propose_block_noalloc(cfg, w, cache, batch, bonus_tokens, seq_lens, max_context, draft_token_ids, drafts_only,
                          hidden_out, stream=None) -> None:
    _check(lib().dflash_propose_block_noalloc(ctypes.byref(cfg), ctypes.byref(w), ctypes.byref(cache), batch,
                                              _ptr(bonus_tokens), _ptr(seq_lens), max_context,
                                              _ptr(draft_token_ids), _ptr(drafts_only), _ptr(hidden_out),
                                              _stream(stream)))


def greedy_verify(batch, num_drafts, draft_tokens, target_tokens, accepted_len, output_tokens, next_bonus,
                  stream=None) -> None:
    _check(lib().dflash_greedy_verify(batch, num_drafts, _ptr(draft_tokens), _ptr(target_tokens),
                                      _ptr(accepted_len), _ptr(output_tokens), _ptr(next_bonus), _stream(stream)))


def greedy_verify_stats(batch, num_drafts, draft_tokens, target_tokens, accepted_len, output_tokens, next_bonus,
                        stats, stream=None) -> None:
    _check(lib().dflash_greedy_verify_stats(batch, num_drafts, _ptr(draft_tokens), _ptr(target_tokens),
                                            _ptr(accepted_len), _ptr(output_tokens), _ptr(next_bonus),
                                            _ptr(stats), _stream(stream)))


def prepare_proposal_inputs(batch, prev_num_drafts, prev_out, vocab, opt_seq_lens, n_rows, row_req, opt_positions,
                            block_table, max_blocks_per_seq, page_size, seq_lens, positions, slot_mapping, bonus,
                            stream=None) -> None:
    _check(lib().dflash_prepare_proposal_inputs(batch, prev_num_drafts, _ptr(prev_out), vocab, _ptr(opt_seq_lens),
                                                n_rows, _ptr(row_req), _ptr(opt_positions), _ptr(block_table),
                                                max_blocks_per_seq, page_size, _ptr(seq_lens), _ptr(positions),
                                                _ptr(slot_mapping), _ptr(bonus), _stream(stream)))


# ----------------------------------------------------------------------------------------
# Convenience objects
# ----------------------------------------------------------------------------------------
class PagedCache:
    """Per-layer K and V caches [num_pages, page_size, KVH, D] plus a block table."""

    def __init__(self, spec, num_pages: int, page_size: int, block_table: torch.Tensor | None = None,
                 device="cuda"):
        dt = storage_dtype(spec)
        shape = (num_pages, page_size, spec.n_kv_heads, spec.head_dim)
        self.k = [torch.zeros(shape, dtype=dt, device=device) for _ in range(spec.n_layers)]
        self.v = [torch.zeros(shape, dtype=dt, device=device) for _ in range(spec.n_layers)]
        self.num_pages, self.page_size = num_pages, page_size
        self.set_block_table(block_table)

    def set_block_table(self, block_table: torch.Tensor | None) -> None:
        self.block_table = block_table
        n = max(1, len(self.k))
        self._k_arr = (_vp * n)(*[t.data_ptr() for t in self.k])
        self._v_arr = (_vp * n)(*[t.data_ptr() for t in self.v])
        bt = block_table
        self.struct = KvCache(self._k_arr, self._v_arr, self.num_pages, self.page_size,
                              None if bt is None else bt.data_ptr(), 0 if bt is None else bt.shape[1])


class Drafter:
    """A drafter's weights on the device, the RoPE table and the fused KV weight."""

    def __init__(self, spec, weights: dict, rope_max_pos: int, device="cuda", stream=None):
        self.spec = spec
        self.cfg = make_config(spec)
        dt = storage_dtype(spec)
        self.w = {k: v.to(device=device, dtype=dt).contiguous() for k, v in weights.items()}
        L = spec.n_layers
        half = spec.head_dim // 2
        self.rope_cos = torch.empty((rope_max_pos, half), dtype=torch.float32, device=device)
        self.rope_sin = torch.empty((rope_max_pos, half), dtype=torch.float32, device=device)
        kvn = L * 2 * spec.n_kv_heads * spec.head_dim
        self.kv_fused = torch.empty((max(kvn, 1), spec.hidden), dtype=dt, device=device)
        self._arrays = {}
        for n in _PER_LAYER:
            ptrs = [self.w[f"layers.{l}.{n}"].data_ptr() for l in range(L)] or [0]
            self._arrays[n] = (_vp * len(ptrs))(*ptrs)
        self.struct = Weights(
            self.w["fc"].data_ptr(), self.w["hidden_norm"].data_ptr(), self.w["embed"].data_ptr(),
            self.w["lm_head"].data_ptr(), self.w["final_norm"].data_ptr(), self.kv_fused.data_ptr(),
            *[self._arrays[n] for n in _PER_LAYER], self.rope_cos.data_ptr(), self.rope_sin.data_ptr(), rope_max_pos)
        build_rope_table(spec.head_dim, spec.rope_theta, rope_max_pos, self.rope_cos, self.rope_sin, stream)
        if L:
            build_fused_kv_weight(self.cfg, self.struct, self.kv_fused, stream)

    # -- workspaces
    def workspace(self, op: int, max_rows_or_batch: int, max_context: int = 0, device="cuda") -> torch.Tensor:
        n = workspace_bytes(self.cfg, op, max_rows_or_batch, max_context)
        if n == 0:
            raise DFlashError(-1, "invalid configuration for workspace sizing")
        return torch.empty(n, dtype=torch.uint8, device=device)

    # -- the three calls
    def inject(self, cache: PagedCache, aux: list, positions, slot_mapping, workspace, stream=None) -> None:
        n = int(positions.shape[0])
        stride = aux[0].stride(0) if n else self.spec.target_hidden
        inject_context_kv(self.cfg, self.struct, cache.struct, aux, stride, n, positions, slot_mapping, workspace,
                          stream)

    def propose(self, cache: PagedCache, bonus, seq_lens, max_context: int, workspace, out=None,
                hidden_out=None, stream=None, cache_ready=None):
        B = int(bonus.shape[0])
        K = self.spec.block_size - 1
        if out is None:
            out = (torch.empty((B, K + 1), dtype=torch.int32, device=bonus.device),
                   torch.empty((B, K), dtype=torch.int32, device=bonus.device))
        if cache_ready is None:
            propose_block(self.cfg, self.struct, cache.struct, B, bonus, seq_lens, max_context, out[0], out[1],
                          hidden_out, workspace, stream)
        else:
            propose_block_after(self.cfg, self.struct, cache.struct, B, bonus, seq_lens, max_context, out[0], out[1],
                                hidden_out, workspace, cache_ready, stream)
        return out

    def propose_noalloc(self, cache: PagedCache, bonus, seq_lens, max_context: int, out=None, hidden_out=None,
                        stream=None):
        """propose() on the library's static device scratch (no workspace)."""
        B = int(bonus.shape[0])
        K = self.spec.block_size - 1
        if out is None:
            out = (torch.empty((B, K + 1), dtype=torch.int32, device=bonus.device),
                   torch.empty((B, K), dtype=torch.int32, device=bonus.device))
        propose_block_noalloc(self.cfg, self.struct, cache.struct, B, bonus, seq_lens, max_context, out[0], out[1],
                              hidden_out, stream)
        return out


def profile_enable(on: bool) -> None:
    _check(lib().dflash_profile_enable(1 if on else 0))


def profile_filter(names=None) -> None:
    """Time only the launches of these kernel names (None: every launch)."""
    _check(lib().dflash_profile_filter(",".join(names).encode() if names else None))


def profile_reset() -> None:
    lib().dflash_profile_reset()


def profile_collect() -> dict:
    """Wait for the recorded launch events; returns {kernel name: (launches, total ms)}."""
    L = lib()
    _check(L.dflash_profile_collect())
    out = {}
    for i in range(L.dflash_profile_count()):
        name, n, ms = ctypes.c_char_p(), ctypes.c_int64(), ctypes.c_double()
        _check(L.dflash_profile_entry(i, ctypes.byref(name), ctypes.byref(n), ctypes.byref(ms)))
        out[name.value.decode()] = (int(n.value), float(ms.value))
    return out


def verify(drafts, target, out=None, stream=None):
    """Greedy verification; returns (accepted_len [B], output_tokens [B, K+1], next_bonus [B])."""
    B, K = drafts.shape
    if out is None:
        out = (torch.empty(B, dtype=torch.int32, device=drafts.device),
               torch.empty((B, K + 1), dtype=torch.int32, device=drafts.device),
               torch.empty(B, dtype=torch.int32, device=drafts.device))
    greedy_verify(B, K, drafts, target, out[0], out[1], out[2], stream)
    return out


def verify_with_stats(drafts, target, stats, out=None, stream=None):
    """Greedy verification that also adds this call's acceptance counters to stats
    (int64 [3]: num_drafts, num_draft_tokens, num_accepted_tokens)."""
    B, K = drafts.shape
    if out is None:
        out = (torch.empty(B, dtype=torch.int32, device=drafts.device),
               torch.empty((B, K + 1), dtype=torch.int32, device=drafts.device),
               torch.empty(B, dtype=torch.int32, device=drafts.device))
    greedy_verify_stats(B, K, drafts, target, out[0], out[1], out[2], stats, stream)
    return out


def prepare(prev_out, vocab, opt_seq_lens, row_req, opt_positions, block_table, page_size, out=None, stream=None):
    """Proposal-input preparation; returns (seq_lens [B], positions [n], slot_mapping [n] int64,
    bonus [B])."""
    B, K1 = prev_out.shape
    n = int(row_req.shape[0])
    dev = prev_out.device
    if out is None:
        out = (torch.empty(B, dtype=torch.int32, device=dev), torch.empty(n, dtype=torch.int32, device=dev),
               torch.empty(n, dtype=torch.int64, device=dev), torch.empty(B, dtype=torch.int32, device=dev))
    prepare_proposal_inputs(B, K1 - 1, prev_out, vocab, opt_seq_lens, n, row_req, opt_positions, block_table,
                            int(block_table.shape[1]), page_size, out[0], out[1], out[2], out[3], stream)
    return out
