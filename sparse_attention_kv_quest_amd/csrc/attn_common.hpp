// Shared description of one attention launch and the view -> slot mapping.
#pragma once
#include "se_internal.hpp"

namespace se {

constexpr float LOG2E = 1.4426950408889634f;

struct AttnArgs {
  const void* q; const void* k; const void* v;
  const int32_t* seq_len; const int32_t* view_idx; const int32_t* view_len;
  float* out; float* lse; float* logits;
  float* part_ml;   // [units][splits][G][2]: running max, running sum
  float* part_o;    // [units][splits][G][Dv]: unnormalised output
  float scale;
  int B, Hq, Hkv, G, Dk, Dv, cap, latent, dtype;
  int k_stride, v_stride;  // elements per K / V row
  int view_cap, gran, gshift, logit_cap, splits;   // gshift = log2(gran) or -1
};

// Number of view slots of a unit: view entries times granularity, or seq_len for the identity view.
__device__ __forceinline__ int view_slot_count(const AttnArgs& a, int unit, int b) {
  if (a.view_idx == nullptr) return min(a.seq_len[b], a.cap);
  return min(a.view_len[unit], a.view_cap) * a.gran;
}

// Cache slot read by view slot `s` of a unit, or -1 if it holds no valid token.
__device__ __forceinline__ int view_token(const AttnArgs& a, int unit, int b, int s) {
  const int len = min(a.seq_len[b], a.cap);
  if (a.view_idx == nullptr) return s < len ? s : -1;
  const int e = s / a.gran, o = s - e * a.gran;
  const int page = a.view_idx[size_t(unit) * a.view_cap + e];
  if (page < 0) return -1;
  const int64_t t = int64_t(page) * a.gran + o;
  return t < len ? int(t) : -1;
}

inline AttnArgs make_attn_args(const se_cache& c, const void* q, const void* k, const void* v,
                               const int32_t* seq_len, const int32_t* view_idx, const int32_t* view_len,
                               int view_cap, int gran, float scale, float* out, float* lse, float* logits,
                               int logit_cap) {
  AttnArgs a{};
  a.q = q; a.k = k; a.v = c.latent ? k : v;
  a.seq_len = seq_len; a.view_idx = view_idx; a.view_len = view_len;
  a.out = out; a.lse = lse; a.logits = logits;
  a.scale = scale;
  a.B = c.batch; a.Hq = c.n_q_heads; a.Hkv = c.n_kv_heads; a.G = c.n_q_heads / c.n_kv_heads;
  a.Dk = c.d_k; a.Dv = c.d_v; a.cap = c.capacity; a.latent = c.latent; a.dtype = c.dtype;
  a.k_stride = c.d_k; a.v_stride = c.latent ? c.d_k : c.d_v;
  a.view_cap = view_idx ? view_cap : 0; a.gran = view_idx ? gran : 1;
  a.gshift = -1;
  for (int sh = 0; sh < 31; ++sh)
    if ((1 << sh) == a.gran) { a.gshift = sh; break; }
  a.logit_cap = logits ? logit_cap : 0;
  return a;
}

bool attn_mfma_supported(const AttnArgs& a);
bool attn_mla_supported(const AttnArgs& a);
int attn_mla_auto_splits(int units, int G, int slots);
se_status launch_attn_mla(const AttnArgs& a, hipStream_t s);
int attn_mfma_auto_splits(int units, int slots);
se_status launch_attn_mfma(const AttnArgs& a, hipStream_t s);

inline bool attn_mfma_eligible(const se_cache& c) {
  return c.dtype == SE_BF16 && !c.latent && (c.d_k == 128 || c.d_k == 64) && c.d_v == c.d_k &&
         c.n_q_heads / c.n_kv_heads <= 16;
}

inline bool attn_mla_eligible(const se_cache& c) {
  return c.dtype == SE_BF16 && c.latent && c.d_k == 576 && c.d_v == 512 && c.n_q_heads / c.n_kv_heads <= 64;
}

}  // namespace se
