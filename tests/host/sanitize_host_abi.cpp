// Host-side paths of the C ABI under AddressSanitizer and UndefinedBehaviorSanitizer:
// the row-budget planner, model validation and destruction, workspace sizing, argument
// rejection before any launch, the miss back-off and the window helper.  Every call here
// returns before anything is enqueued, so no GPU is needed.  Exits non-zero on a failed
// check; the sanitizers abort on a memory or undefined-behaviour error.
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <vector>

#include "spec_verify.h"

static int failures = 0;
#define CHECK(c)                                                          \
  do {                                                                    \
    if (!(c)) {                                                           \
      std::fprintf(stderr, "check failed at line %d: %s\n", __LINE__, #c); \
      ++failures;                                                         \
    }                                                                     \
  } while (0)

static void* const FAKE = reinterpret_cast<void*>(0x1000);   // never dereferenced

struct Desc {
  spec_model_desc d{};
  std::vector<int32_t> kinds;
  std::vector<spec_layer_weights> lw;
};

static Desc make_desc(int n_layers, int dtype, int hidden, int vocab, int gdn_every = 0) {
  Desc x;
  x.kinds.resize(n_layers > 0 ? n_layers : 1);
  x.lw.resize(n_layers > 0 ? n_layers : 1);
  for (int i = 0; i < n_layers; ++i) {
    x.kinds[i] = (gdn_every && i % gdn_every != gdn_every - 1) ? SPEC_LAYER_GDN : SPEC_LAYER_ATTN;
    x.lw[i] = spec_layer_weights{(const float*)FAKE, FAKE, FAKE, (const float*)FAKE, FAKE, FAKE, FAKE};
  }
  spec_model_desc& d = x.d;
  d.n_layers = n_layers;
  d.hidden = hidden;
  d.n_q_heads = 4; d.n_kv_heads = 2; d.head_dim = 128;
  d.ffn = 512; d.vocab = vocab; d.dtype = dtype;
  d.layer_kind = x.kinds.data();
  d.gdn_heads = gdn_every ? 2 : 0; d.gdn_dim = gdn_every ? 128 : 0;
  d.rms_eps = 1e-6f; d.rope_theta = 1e4f; d.kv_block = SPEC_KV_BLOCK; d.attn_chunk = 0;
  d.embed = FAKE; d.lm_head = FAKE; d.final_norm = (const float*)FAKE;
  d.layers = x.lw.data();
  return x;
}

int main() {
  // planner: the closed form, and its errors
  for (int k = 0; k <= 16; ++k)
    for (int budget = 0; budget <= 64; ++budget)
      for (int lanes = 1; lanes <= 64; ++lanes) {
        const int rows = budget == 0 ? 8 : budget;
        int want = rows / lanes - 1;
        want = want < 0 ? 0 : (want > k ? k : want);
        CHECK(spec_plan_drafts(k, budget, lanes) == want);
      }
  CHECK(spec_plan_drafts(3, 8, 0) == SPEC_E_INVAL);
  CHECK(spec_plan_drafts(-1, 8, 1) == SPEC_E_INVAL);
  for (int s = 1; s >= -7; --s) CHECK(spec_status_string(s) != nullptr);

  // models: valid and invalid descriptions, created and destroyed many times
  for (int rep = 0; rep < 50; ++rep) {
    for (int dtype : {SPEC_F32, SPEC_BF16}) {
      for (int gdn : {0, 4}) {
        Desc x = make_desc(4, dtype, 256, 1024, gdn);
        spec_model* m = nullptr;
        CHECK(spec_model_create(&x.d, &m) == SPEC_OK && m);
        for (int lanes = 1; lanes <= SPEC_MAX_LANES; lanes += 7)
          for (int cols = 1; cols <= SPEC_MAX_COLS; cols += 5)
            CHECK(spec_workspace_bytes(m, lanes, cols, 40) > 0);
        CHECK(spec_workspace_bytes(m, 0, 4, 4) == SPEC_E_INVAL);
        CHECK(spec_workspace_bytes(m, 2, SPEC_MAX_COLS + 1, 4) == SPEC_E_INVAL);
        // rounds refused before any launch
        int32_t cols[SPEC_MAX_LANES];
        for (int i = 0; i < SPEC_MAX_LANES; ++i) cols[i] = 4;
        int32_t kvh[2] = {61, 0};
        spec_round r{};
        r.lanes = 2; r.cols_host = cols; r.tokens = (const int32_t*)FAKE; r.kv_len = (int32_t*)FAKE;
        r.block_table = (const int32_t*)FAKE; r.max_blocks = 4; r.k_pool = FAKE; r.v_pool = FAKE; r.n_blocks = 16;
        r.gdn_state = (float*)FAKE; r.workspace = reinterpret_cast<void*>(0x100000); r.workspace_bytes = 16;
        CHECK(spec_verify_round(m, &r, nullptr) == SPEC_E_WORKSPACE);
        r.kv_len_host = kvh;
        CHECK(spec_verify_round(m, &r, nullptr) == SPEC_E_RANGE);
        r.kv_len_host = nullptr;
        r.lanes = 0;
        CHECK(spec_verify_round(m, &r, nullptr) == SPEC_E_INVAL);
        CHECK(spec_accept(m, &r, (int32_t*)FAKE, (int32_t*)FAKE, nullptr, nullptr) == SPEC_E_INVAL);
        CHECK(spec_commit(m, &r, (const int32_t*)FAKE, nullptr) == SPEC_E_INVAL);
        r.lanes = 5; 
        for (int i = 0; i < 5; ++i) cols[i] = 16;   // 80 rows
        CHECK(spec_verify_round(m, &r, nullptr) == SPEC_E_INVAL);
        r.lanes = 2; cols[0] = cols[1] = 4;
        r.mode = SPEC_SAMPLED;                      // no q_probs
        CHECK(spec_verify_round(m, &r, nullptr) == SPEC_E_INVAL);
        r.mode = SPEC_GREEDY;
        if (gdn) {
          r.gdn_state = nullptr;
          CHECK(spec_verify_round(m, &r, nullptr) == SPEC_E_UNSUPPORTED);
        }
        CHECK(spec_verify_head(m, &r, nullptr, nullptr) == SPEC_E_INVAL);
        CHECK(spec_verify_head_noalloc(m, &r, nullptr, (int32_t*)FAKE, (int32_t*)FAKE, nullptr, nullptr) ==
              SPEC_E_INVAL);
        CHECK(spec_profile_enable(m, 99, 1) == SPEC_E_INVAL);
        spec_model_destroy(m);
      }
    }
    Desc bad = make_desc(2, SPEC_BF16, 200, 1024);   // bf16 hidden must be a multiple of 256
    spec_model* m = nullptr;
    CHECK(spec_model_create(&bad.d, &m) == SPEC_E_UNSUPPORTED && m == nullptr);
    bad = make_desc(2, SPEC_BF16, 256, 1000);        // vocab not a multiple of 16
    CHECK(spec_model_create(&bad.d, &m) == SPEC_E_INVAL && m == nullptr);
  }
  spec_model_destroy(nullptr);

  // a head-only round larger than the static scratch is refused before any device call
  {
    Desc x = make_desc(0, SPEC_BF16, 256, 1 << 20);
    spec_model* m = nullptr;
    CHECK(spec_model_create(&x.d, &m) == SPEC_OK);
    int32_t cols[8] = {8, 8, 8, 8, 8, 8, 8, 8};
    spec_round r{};
    r.lanes = 8; r.cols_host = cols; r.tokens = (const int32_t*)FAKE; r.kv_len = (int32_t*)FAKE;
    CHECK(spec_verify_head_noalloc(m, &r, FAKE, (int32_t*)FAKE, (int32_t*)FAKE, nullptr, nullptr) == SPEC_E_SCRATCH);
    spec_model_destroy(m);
  }

  // miss back-off: long random pass sequences stay in range
  {
    spec_backoff st[SPEC_MAX_LANES];
    int32_t drafts[SPEC_MAX_LANES], kept[SPEC_MAX_LANES];
    unsigned seed = 12345u;
    auto rnd = [&]() { seed = seed * 1664525u + 1013904223u; return seed >> 8; };
    for (int n = 1; n <= SPEC_MAX_LANES; n += 9) {
      CHECK(spec_backoff_init(st, n) == SPEC_OK);
      for (int call = 0; call < 300; ++call) {
        const int sp = spec_backoff_call(st, n, 7, (int)(rnd() % 70), drafts);
        CHECK(sp == 0 || sp == 1);
        for (int pass = 0; pass < 8; ++pass) {
          for (int i = 0; i < n; ++i) kept[i] = (rnd() % 5 == 0) ? (int)(rnd() % 4) : 0;
          CHECK(spec_backoff_pass(st, n, kept, sp) == SPEC_OK);
          for (int i = 0; i < n; ++i)
            CHECK(st[i].wait_len >= 16 && st[i].wait_len <= 256 && st[i].wait_left >= 0 && st[i].miss_run >= 0 &&
                  st[i].miss_run < 4);
        }
      }
    }
    CHECK(spec_backoff_init(st, 0) == SPEC_E_INVAL);
    CHECK(spec_backoff_call(st, SPEC_MAX_LANES + 1, 7, 8, drafts) == SPEC_E_INVAL);
    CHECK(spec_backoff_pass(nullptr, 1, kept, 1) == SPEC_E_INVAL);
  }

  // window helper and the validation of the drafter and count calls
  CHECK(spec_window_live_block(-1, 8) == SPEC_E_INVAL);
  CHECK(spec_window_live_block(8192, 1024) == (8192 - 1024 + 1) / 64 * 4);
  CHECK(spec_ngram_draft(nullptr, (const int32_t*)FAKE, 2, 64, 3, 3, 1, (int32_t*)FAKE, (int32_t*)FAKE, nullptr) ==
        SPEC_E_INVAL);
  CHECK(spec_history_append((int32_t*)FAKE, (int32_t*)FAKE, 0, 64, (const int32_t*)FAKE, (const int32_t*)FAKE, 16,
                            nullptr) == SPEC_E_INVAL);
  CHECK(spec_counts_add((int32_t*)FAKE, 0, 2, (const int32_t*)FAKE, (const int32_t*)FAKE, 16, nullptr) ==
        SPEC_E_INVAL);
  CHECK(spec_packed_weight_bytes(151936, 5120) == (int64_t)151936 * 5120 * 2);
  CHECK(spec_pack_weight(FAKE, FAKE, 16, 256, nullptr) == SPEC_E_INVAL);

  if (failures) {
    std::fprintf(stderr, "%d checks failed\n", failures);
    return 1;
  }
  std::printf("host ABI checks passed under the sanitizers\n");
  return 0;
}
