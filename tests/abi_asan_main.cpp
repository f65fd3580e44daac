// Host-side checks of the C ABI under AddressSanitizer (built by
// block_diffusion_drafting_concat_amd/build.py build_asan_driver(): api.cpp and profile.cpp with
// host-only -fsanitize=address, linked with the kernel objects). Every call here stays in host
// code: argument validation, workspace planning, status strings, the last-error string and the
// profiling registry. Dummy device pointers are never dereferenced: a call that got past its
// validation would reach the HIP runtime, which has no device here and returns an error that
// the checks below would see. Exit status 0 when every check holds.
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include <vector>

#include "../include/dflash.h"

static int g_failed = 0;
#define CHECK(cond)                                                             \
  do {                                                                          \
    if (!(cond)) {                                                              \
      fprintf(stderr, "check failed at line %d: %s (last error: %s)\n", __LINE__, #cond, \
              dflash_last_error());                                             \
      ++g_failed;                                                               \
    }                                                                           \
  } while (0)

static dflash_config qwen3() {
  dflash_config c{};
  c.hidden = 4096, c.n_layers = 5, c.n_q_heads = 32, c.n_kv_heads = 8, c.head_dim = 128;
  c.intermediate = 12288, c.vocab = 151936, c.n_aux = 5, c.target_hidden = 4096, c.block_size = 16;
  c.mask_token_id = 151935, c.rms_eps = 1e-6f, c.dtype = DFLASH_BF16;
  return c;
}

static void *dummy(uintptr_t x) { return reinterpret_cast<void *>(x); }

int main() {
  // status strings and the thread-local error string
  CHECK(strcmp(dflash_status_string(DFLASH_OK), "ok") == 0);
  CHECK(strcmp(dflash_status_string(DFLASH_ERR_WORKSPACE_TOO_SMALL), "workspace too small") == 0);
  CHECK(strcmp(dflash_status_string(12345), "unknown status") == 0);

  // invalid configurations: workspace sizing returns 0, calls return an error with a message
  dflash_config bad = qwen3();
  bad.head_dim = 96;
  CHECK(dflash_workspace_bytes(&bad, DFLASH_OP_PROPOSE, 1, 128) == 0);
  CHECK(dflash_propose_block(&bad, nullptr, nullptr, 1, nullptr, nullptr, 0, nullptr, nullptr, nullptr, nullptr, 0,
                             nullptr) == DFLASH_ERR_UNSUPPORTED);
  CHECK(strlen(dflash_last_error()) > 0);
  CHECK(dflash_workspace_bytes(nullptr, DFLASH_OP_INJECT, 1, 0) == 0);
  bad = qwen3();
  bad.n_q_heads = 30;
  CHECK(dflash_inject_context_kv(&bad, nullptr, nullptr, nullptr, 4096, 1, nullptr, nullptr, nullptr, 0, nullptr) ==
        DFLASH_ERR_INVALID_ARGUMENT);

  // workspace plans over many sizes (the planner's arithmetic runs under the sanitizer)
  dflash_config c = qwen3();
  size_t prev = 0;
  for (int rows : {1, 16, 64, 65, 4096, 10000}) {
    const size_t n = dflash_workspace_bytes(&c, DFLASH_OP_INJECT, rows, 0);
    CHECK(n > 0 && n >= prev);
    prev = n;
  }
  for (int b : {1, 32, 128}) CHECK(dflash_workspace_bytes(&c, DFLASH_OP_PROPOSE, b, 32768) > 0);
  CHECK(dflash_workspace_bytes(&c, 7, 1, 0) == 0);

  // empty calls succeed before touching any pointer
  CHECK(dflash_propose_block(&c, nullptr, nullptr, 0, nullptr, nullptr, 0, nullptr, nullptr, nullptr, nullptr, 0,
                             nullptr) == DFLASH_OK);
  CHECK(strlen(dflash_last_error()) == 0);
  CHECK(dflash_inject_context_kv(&c, nullptr, nullptr, nullptr, 4096, 0, nullptr, nullptr, nullptr, 0, nullptr) ==
        DFLASH_OK);

  // dummy weights and cache: every pointer non-NULL, none dereferenced
  std::vector<const void *> layer(c.n_layers, dummy(0x100000));
  std::vector<void *> kv(c.n_layers, dummy(0x200000));
  dflash_weights w{};
  w.fc = w.hidden_norm = w.embed = w.lm_head = w.final_norm = w.kv_fused = dummy(0x300000);
  w.in_norm = w.wq = w.wk = w.wv = w.q_norm = w.k_norm = w.wo = w.post_norm = w.w_gate = w.w_up = w.w_down =
      layer.data();
  w.rope_cos = w.rope_sin = static_cast<const float *>(dummy(0x400000));
  w.rope_max_pos = 40000;
  dflash_kv_cache cache{kv.data(), kv.data(), 4096, 16, static_cast<const int32_t *>(dummy(0x500000)), 256};
  std::vector<const void *> aux(c.n_aux, dummy(0x600000));
  const int32_t *pos = static_cast<const int32_t *>(dummy(0x700000));
  const int64_t *slots = static_cast<const int64_t *>(dummy(0x800000));
  // workspace too small for a chunk of an injection (one chunk or several): refused before any
  // launch (a launch here, with no device, would return a HIP error instead). The query is the
  // maximum over every chunk size up to its row count, so a call can need less than it: the
  // workspaces below are too small for any chunk of these calls.
  const size_t need16 = dflash_workspace_bytes(&c, DFLASH_OP_INJECT, 16, 0);
  for (int rows : {16, 4096, 4196, 12289}) {
    for (size_t ws : {(size_t)1, need16}) {
      if (rows <= 16 && ws == need16) continue;  // enough for a 16-row call
      CHECK(dflash_inject_context_kv(&c, &w, &cache, aux.data(), 4096, rows, pos, slots, dummy(0x900000), ws,
                                     nullptr) == DFLASH_ERR_WORKSPACE_TOO_SMALL);
    }
  }
  CHECK(dflash_inject_context_kv(&c, &w, &cache, aux.data(), 4095, 16, pos, slots, dummy(0x900000), 1 << 30,
                                 nullptr) == DFLASH_ERR_INVALID_ARGUMENT);  // stride below target_hidden
  const size_t pneed = dflash_workspace_bytes(&c, DFLASH_OP_PROPOSE, 4, 2048);
  int32_t *out = static_cast<int32_t *>(dummy(0xA00000));
  CHECK(dflash_propose_block(&c, &w, &cache, 4, pos, pos, 2048, out, out, nullptr, dummy(0x900000), pneed - 1,
                             nullptr) == DFLASH_ERR_WORKSPACE_TOO_SMALL);
  w.wq = nullptr;
  CHECK(dflash_propose_block(&c, &w, &cache, 4, pos, pos, 2048, out, out, nullptr, dummy(0x900000), pneed,
                             nullptr) == DFLASH_ERR_INVALID_ARGUMENT);

  // verification and preparation argument checks
  CHECK(dflash_greedy_verify(0, 7, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr) == DFLASH_OK);
  CHECK(dflash_greedy_verify(1, 64, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr) == DFLASH_ERR_UNSUPPORTED);
  CHECK(dflash_greedy_verify(1, 7, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr) ==
        DFLASH_ERR_INVALID_ARGUMENT);
  CHECK(dflash_greedy_verify_stats(1, 7, pos, pos, out, out, out, nullptr, nullptr) == DFLASH_ERR_INVALID_ARGUMENT);
  CHECK(dflash_prepare_proposal_inputs(1, 3, nullptr, 10, nullptr, 0, nullptr, nullptr, nullptr, 4, 0, nullptr,
                                       nullptr, nullptr, nullptr, nullptr) == DFLASH_ERR_INVALID_ARGUMENT);
  CHECK(dflash_build_rope_table(63, 1e6, 10, nullptr, nullptr, nullptr) == DFLASH_ERR_INVALID_ARGUMENT);

  // profiling registry (host only: nothing is enabled, so no event is created)
  const char *long_list = "gemm.qkv,gemm.o,gemm.gate_up,gemm.down,attn_partial,attn_merge,a,b,c,d,e,f,g,h";
  CHECK(dflash_profile_filter(long_list) == DFLASH_OK);
  CHECK(dflash_profile_filter("") == DFLASH_OK);
  CHECK(dflash_profile_filter(nullptr) == DFLASH_OK);
  dflash_profile_reset();
  CHECK(dflash_profile_collect() == DFLASH_OK);
  CHECK(dflash_profile_count() == 0);

  if (g_failed) fprintf(stderr, "%d checks failed\n", g_failed);
  else printf("abi host checks passed\n");
  return g_failed ? 1 : 0;
}
