// Host-side driver of the libse C ABI, built with AddressSanitizer and
// UndefinedBehaviorSanitizer on the host code: every entry point is called with
// arguments the host validation must reject (nothing reaches the GPU), and the
// host computations (per-layer budgets, prefix matching, workspace sizes) run on
// many random inputs.  Exit status 0 when every call returns what the header
// promises; a sanitizer report aborts the run.
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <random>
#include <vector>

#include "se.h"

static int failures = 0;

#define EXPECT(expr, want)                                                                             \
  do {                                                                                                 \
    const int got_ = int(expr);                                                                        \
    if (got_ != int(want)) {                                                                           \
      std::fprintf(stderr, "%s:%d: %s returned %d, expected %d\n", __FILE__, __LINE__, #expr, got_,   \
                   int(want));                                                                         \
      ++failures;                                                                                      \
    }                                                                                                  \
  } while (0)

// Aligned, never dereferenced addresses: validation fails before any launch.
static void* const A = reinterpret_cast<void*>(0x10000);
static void* const M = reinterpret_cast<void*>(0x10008);   // 8-byte aligned only
static float* const F = reinterpret_cast<float*>(0x10000);
static int32_t* const I = reinterpret_cast<int32_t*>(0x10000);
static uint8_t* const U = reinterpret_cast<uint8_t*>(0x10000);

static se_cache cache(int b, int hq, int hkv, int dk, int dv, int cap, se_dtype dt = SE_BF16, int latent = 0) {
  se_cache c;
  std::memset(&c, 0, sizeof(c));
  c.batch = b; c.n_q_heads = hq; c.n_kv_heads = hkv; c.d_k = dk; c.d_v = dv; c.capacity = cap;
  c.dtype = dt; c.latent = latent;
  return c;
}

static void cache_checks() {
  const se_cache bad[] = {cache(0, 8, 2, 128, 128, 64), cache(2, 8, 3, 128, 128, 64), cache(2, 8, 2, 96, 96, 64),
                          cache(2, 8, 2, 128, 64, 64), cache(2, 8, 2, 128, 128, 0), cache(2, 8, 2, 576, 512, 64, SE_BF16, 1),
                          cache(2, 260, 2, 128, 128, 64)};
  for (const se_cache& c : bad) {
    EXPECT(se_kv_append(&c, A, A, A, A, nullptr, I, nullptr), SE_ERR_SHAPE);
    EXPECT(se_sparse_decode_attn(&c, A, A, A, I, nullptr, nullptr, 0, 1, 0.1f, F, nullptr, nullptr, 0, 0, A, 1 << 20,
                                 nullptr), SE_ERR_SHAPE);
    EXPECT(se_workspace_bytes(SE_OP_ATTN, &c, 64, 0), 0);
  }
  se_cache dt = cache(2, 8, 2, 128, 128, 64);
  dt.dtype = static_cast<se_dtype>(7);
  EXPECT(se_kv_append(&dt, A, A, A, A, nullptr, I, nullptr), SE_ERR_DTYPE);
  EXPECT(se_kv_append(nullptr, A, A, A, A, nullptr, I, nullptr), SE_ERR_NULL);
}

static void entry_point_checks() {
  const se_cache c = cache(2, 8, 2, 128, 128, 1024);
  // append and page metadata
  EXPECT(se_kv_append(&c, nullptr, A, A, A, nullptr, I, nullptr), SE_ERR_NULL);
  EXPECT(se_kv_append(&c, M, A, A, A, nullptr, I, nullptr), SE_ERR_ALIGN);
  EXPECT(se_kv_append_meta(&c, A, A, A, A, nullptr, I, A, nullptr, 16, nullptr), SE_ERR_NULL);
  EXPECT(se_page_meta_update(&c, A, A, A, I, 0, 0, nullptr), SE_ERR_SHAPE);
  // Quest
  EXPECT(se_quest_select(&c, A, A, A, I, 16, 0, I, I, nullptr, A, 1 << 20, nullptr), SE_ERR_BUDGET);
  EXPECT(se_quest_select(&c, A, A, A, I, 16, 8, I, I, nullptr, A, 4, nullptr), SE_ERR_WORKSPACE);
  EXPECT(se_quest_append_select(&c, A, A, A, A, A, I, A, A, 16, 8, nullptr, I, nullptr, A, 1 << 20, nullptr),
         SE_ERR_NULL);
  EXPECT(se_quest_decode_step(&c, A, A, A, A, A, I, A, A, 16, 8, 0.1f, F, F, I, nullptr, nullptr, A, 1 << 24,
                              nullptr), SE_ERR_NULL);   // view without view_len
  EXPECT(se_quest_decode_step(&c, A, A, A, A, A, I, A, A, 16, 0, 0.1f, F, F, nullptr, nullptr, nullptr, A, 1 << 24,
                              nullptr), SE_ERR_BUDGET);
  EXPECT(se_quest_decode_step(&c, A, A, A, A, A, I, A, A, 16, 8, -1.f, F, F, nullptr, nullptr, nullptr, A, 1 << 24,
                              nullptr), SE_ERR_SHAPE);
  EXPECT(se_quest_decode_step(&c, A, A, A, A, A, I, A, A, 16, 8, 0.1f, F, F, nullptr, nullptr, nullptr, A, 16,
                              nullptr), SE_ERR_WORKSPACE);
  // the FP8 decode step
  EXPECT(se_quest_decode_step_fp8(&c, A, A, A, U, nullptr, A, A, I, A, A, 16, 8, 0.1f, F, F, nullptr, nullptr,
                                  nullptr, A, 1 << 24, nullptr), SE_ERR_NULL);   // no V scales
  EXPECT(se_quest_decode_step_fp8(&c, A, A, A, U, U, A, A, I, A, A, 16, 0, 0.1f, F, F, nullptr, nullptr, nullptr, A,
                                  1 << 24, nullptr), SE_ERR_BUDGET);
  EXPECT(se_quest_decode_step_fp8(&c, A, A, A, U, U, A, A, I, A, A, 16, 8, 0.f, F, F, nullptr, nullptr, nullptr, A,
                                  1 << 24, nullptr), SE_ERR_SHAPE);
  EXPECT(se_quest_decode_step_fp8(&c, A, A, A, U, U, A, A, I, A, A, 16, 8, 0.1f, F, F, nullptr, nullptr, nullptr, A,
                                  16, nullptr), SE_ERR_WORKSPACE);
  {
    const se_cache wide = cache(2, 64, 2, 128, 128, 1024);   // 32 heads per KV head
    EXPECT(se_quest_decode_step_fp8(&wide, A, A, A, U, U, A, A, I, A, A, 16, 8, 0.1f, F, F, nullptr, nullptr,
                                    nullptr, A, 1 << 26, nullptr), SE_ERR_UNSUPPORTED);
  }
  // attention
  EXPECT(se_sparse_decode_attn(&c, A, A, A, I, I, nullptr, 8, 16, 0.1f, F, nullptr, nullptr, 0, 0, A, 1 << 20,
                               nullptr), SE_ERR_NULL);
  EXPECT(se_sparse_decode_attn(&c, A, A, A, I, nullptr, nullptr, 0, 1, 0.1f, F, nullptr, F, 0, 0, A, 1 << 20,
                               nullptr), SE_ERR_SHAPE);
  EXPECT(se_sparse_decode_attn(&c, A, A, A, I, nullptr, nullptr, 0, 1, 0.1f, F, nullptr, nullptr, 0, 257, A,
                               1 << 20, nullptr), SE_ERR_SHAPE);
  EXPECT(se_sparse_decode_attn_noalloc(&c, M, A, A, I, nullptr, nullptr, 0, 1, 0.1f, F, nullptr, nullptr, 0, 0,
                                       nullptr), SE_ERR_ALIGN);
  const se_cache big = cache(64, 32, 4, 128, 128, 16384);
  EXPECT(se_sparse_decode_attn_noalloc(&big, A, A, A, I, nullptr, nullptr, 0, 1, 0.1f, F, nullptr, nullptr, 0, 256,
                                       nullptr), SE_ERR_WORKSPACE);
  EXPECT(se_kv_append_decode_attn(&c, A, A, A, A, A, nullptr, I, nullptr, nullptr, 0, 1, 0.1f, F, nullptr, nullptr,
                                  0, 0, nullptr, 0, nullptr), SE_ERR_WORKSPACE);
  // SnapKV
  const se_cache out = cache(2, 8, 2, 128, 128, 100);
  EXPECT(se_snapkv_score_compact(&c, A, A, A, 500, 16, 6, 100, 0.1f, &out, A, A, I, nullptr, nullptr, A, 1 << 26,
                                 nullptr), SE_ERR_BUDGET);   // even pool kernel
  EXPECT(se_snapkv_score_compact(&c, A, A, A, 500, 500, 7, 100, 0.1f, &out, A, A, I, nullptr, nullptr, A, 1 << 26,
                                 nullptr), SE_ERR_BUDGET);   // window not below the prompt
  EXPECT(se_snapkv_score_compact(&c, A, A, A, 500, 16, 7, 200, 0.1f, &out, A, A, I, nullptr, nullptr, A, 1 << 26,
                                 nullptr), SE_ERR_BUDGET);   // output capacity below the budget
  const se_cache wrong = cache(2, 8, 1, 128, 128, 200);
  EXPECT(se_snapkv_score_compact(&c, A, A, A, 500, 16, 7, 100, 0.1f, &wrong, A, A, I, nullptr, nullptr, A, 1 << 26,
                                 nullptr), SE_ERR_SHAPE);
  // H2O
  EXPECT(se_h2o_accumulate_evict(&c, F, F, 512, I, I, F, 10, 600, 500, I, nullptr), SE_ERR_SHAPE);   // logit_cap < cap
  EXPECT(se_h2o_accumulate_evict(&c, F, F, 1024, I, I, F, 10, 600, 500, I, nullptr), SE_ERR_BUDGET);
  EXPECT(se_h2o_decode_step(&c, A, A, A, A, A, I, I, I, F, 10, 60, 20, 0.1f, F, nullptr, I, A, 1 << 26, nullptr),
         SE_ERR_SHAPE);   // slot_in aliasing evict_out
  EXPECT(se_h2o_decode_step(&c, A, A, A, A, A, nullptr, I, I, F, -1, 60, 20, 0.1f, F, nullptr, I, A, 1 << 26,
                            nullptr), SE_ERR_SHAPE);
  EXPECT(se_h2o_decode_step(&c, A, A, A, A, A, nullptr, I, I, F, 10, 60, 20, 0.1f, F, nullptr, I, A, 64, nullptr),
         SE_ERR_WORKSPACE);
  EXPECT(se_h2o_prefill_init(&c, A, A, A, 900, 600, 500, 0.1f, &c, A, A, I, F, nullptr, A, 1 << 26, nullptr),
         SE_ERR_BUDGET);
  // OmniKV, StreamingLLM, FP8, Chain Cache
  EXPECT(se_omnikv_topk(&c, F, F, 100, I, 101, I, I, nullptr, A, 1 << 20, nullptr), SE_ERR_BUDGET);
  EXPECT(se_streaming_view(&c, I, 0, 0, I, I, 8, 0, nullptr), SE_ERR_BUDGET);
  EXPECT(se_streaming_view(&c, I, 4, 4, I, I, 7, 0, nullptr), SE_ERR_BUDGET);
  EXPECT(se_kv_quantize_fp8(&c, A, A, I, A, A, nullptr, U, nullptr, nullptr, 0, nullptr), SE_ERR_NULL);
  EXPECT(se_chain_remap(&c, I, 0, I, 8, I, I, nullptr), SE_ERR_SHAPE);
  EXPECT(se_chain_append_positions(&c, I, I, I, -1, nullptr), SE_ERR_SHAPE);
  EXPECT(se_chain_append_positions(&c, I, I, I, 0, nullptr), SE_OK);   // nothing to do, nothing launched
  EXPECT(se_workspace_init(nullptr, 256, nullptr), SE_ERR_NULL);
  EXPECT(se_workspace_init(M, 256, nullptr), SE_ERR_ALIGN);
  EXPECT(se_workspace_init(nullptr, 0, nullptr), SE_OK);
}

static void budget_schedule_checks(std::mt19937& rng) {
  std::vector<int32_t> b(4096);
  EXPECT(se_pyramid_budgets(0, 10, 5, b.data()), SE_ERR_SHAPE);
  EXPECT(se_pyramid_budgets(4, 10, 11, b.data()), SE_ERR_BUDGET);
  EXPECT(se_pyramid_budgets(4, 10, 5, nullptr), SE_ERR_NULL);
  for (int it = 0; it < 20000; ++it) {
    const int n = 1 + int(rng() % 4096);
    const int avg = int(rng() % (it % 2 ? 200000 : 1000));
    const int mn = avg ? int(rng() % (avg + 1)) : 0;
    if (se_pyramid_budgets(n, avg, mn, b.data()) != SE_OK) { ++failures; continue; }
    long long total = 0;
    for (int l = 0; l < n; ++l) {
      total += b[l];
      if (l > 0 && b[l] > b[l - 1]) { ++failures; break; }
    }
    if (total != (long long)n * avg) ++failures;
  }
}

static void prefix_match_checks(std::mt19937& rng) {
  int32_t sess = 0, len = 0;
  EXPECT(se_chain_match(nullptr, 0, nullptr, nullptr, 0, &sess, &len), SE_OK);
  EXPECT(sess, -1);
  EXPECT(se_chain_match(nullptr, 3, nullptr, nullptr, 0, &sess, &len), SE_ERR_NULL);
  for (int it = 0; it < 5000; ++it) {
    const int nt = int(rng() % 64), np = int(rng() % 6);
    std::vector<int32_t> toks(nt);
    for (auto& t : toks) t = int(rng() % 3);
    std::vector<std::vector<int32_t>> pre(np);
    std::vector<const int32_t*> ptrs(np);
    std::vector<int32_t> lens(np);
    for (int s = 0; s < np; ++s) {
      const int n = int(rng() % 70);
      pre[s].resize(n);
      for (int i = 0; i < n; ++i) pre[s][i] = (i < nt && rng() % 8) ? toks[i] : int(rng() % 3);
      ptrs[s] = n ? pre[s].data() : nullptr;
      lens[s] = n;
    }
    if (se_chain_match(toks.data(), nt, ptrs.data(), lens.data(), np, &sess, &len) != SE_OK) { ++failures; continue; }
    int best = -1, best_len = 0;   // a session matches when its whole prefix starts the tokens
    for (int s = 0; s < np; ++s) {
      if (lens[s] > nt) continue;
      bool ok = true;
      for (int i = 0; i < lens[s] && ok; ++i) ok = pre[s][i] == toks[i];
      if (ok && (best < 0 || lens[s] > best_len)) { best = s; best_len = lens[s]; }
    }
    if (sess != best || len != (best < 0 ? 0 : best_len)) ++failures;
  }
}

static void workspace_size_checks(std::mt19937& rng) {
  for (int it = 0; it < 20000; ++it) {
    const int hkv = 1 + int(rng() % 8);
    const se_cache c = cache(1 + int(rng() % 64), hkv * (1 + int(rng() % 16)), hkv, (rng() % 2) ? 128 : 64,
                             0, 1 + int(rng() % 200000), (rng() % 2) ? SE_BF16 : SE_F32);
    se_cache cc = c;
    cc.d_v = cc.d_k;
    for (int op = 0; op <= 10; ++op) (void)se_workspace_bytes(op, &cc, int(rng() % 70000) - 5, int(rng() % 300) - 5);
  }
  for (int st = -20; st <= 5; ++st)
    if (se_status_string(st) == nullptr) ++failures;
}

int main() {
  std::mt19937 rng(1234);
  if (se_abi_version() < 1) ++failures;
  cache_checks();
  entry_point_checks();
  budget_schedule_checks(rng);
  prefix_match_checks(rng);
  workspace_size_checks(rng);
  if (failures) {
    std::fprintf(stderr, "%d check(s) failed\n", failures);
    return 1;
  }
  std::printf("abi driver: all checks passed\n");
  return 0;
}
