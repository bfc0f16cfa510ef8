// Shared description of one attention launch and the view -> slot mapping.
#pragma once
#include "se_internal.hpp"

namespace se {

constexpr float LOG2E = 1.4426950408889634f;
constexpr int ATTN_MAX_HG = 2;          // head groups of one unit launched as separate blocks (MLA, G <= 64)
constexpr int ATTN_MAX_SPLITS = 256;
constexpr size_t ATTN_FUSED_MERGE_BYTES = 64 << 10;   // partial output bytes per unit merged in-kernel

struct AttnArgs {
  const void* q; const void* k; const void* v;
  const int32_t* seq_len; const int32_t* view_idx; const int32_t* view_len;
  float* out; float* lse; float* logits;
  float* part_ml;   // [units][splits][G][2]: running max, running sum
  float* part_o;    // [units][splits][G][Dv]: unnormalised output
  int* counters;    // [units][ATTN_MAX_HG] split completion tickets, zero between calls
  int fused;        // splits > 1 and the last block of a unit merges them (else the combine kernel)
  const uint8_t* k_scale;   // FP8 rows (fp8 != 0): one E8M0 scale byte per K / V row, [units][cap]
  const uint8_t* v_scale;
  int fp8;
  float scale;
  int B, Hq, Hkv, G, Dk, Dv, cap, latent, dtype;
  int k_stride, v_stride;  // elements per K / V row
  int view_cap, gran, gshift, logit_cap, splits;   // gshift = log2(gran) or -1
  // Fused append (app != 0): before attending, row (b, h) of k_new / v_new goes to
  // the cache by se_kv_append's rule (slot[b][h] if slot is given and >= 0, else
  // slot seq_len[b]; a slot at or past the capacity is dropped; seq_len[b] grows
  // by one unless slot[b][0] >= 0).  The launch reads that row from k_new / v_new,
  // one block per unit writes it into k_w / v_w, and the block holding the last
  // ticket of the batch row (row_ctr[b], taken after its tiles, long after it read
  // the old length) stores the new length into seq_len_w.
  const void* k_new; const void* v_new; void* k_w; void* v_w;
  const int32_t* slot; int32_t* seq_len_w; int* row_ctr; int app;
  // In-launch page selection (sel != 0, the Quest decode step): the row at slot
  // seq_len[b] was appended by the preceding scoring launch, so the attention runs
  // over seq_len[b] + 1 slots (capped at the capacity); every block selects its
  // unit's top view_cap pages from sel_score [units][sel_ncp] into its LDS view
  // cache (the rule of the separate top-k launch); split 0 writes the view to
  // sel_view / sel_vlen when they are given; the new length is stored as for app.
  const float* sel_score; int sel_ncp; int32_t* sel_view; int32_t* sel_vlen; int sel;
  // H2O decode step (h2o != 0, with app, the identity view and one split): the
  // logits stay in LDS and, after the attention, the block runs the unit's
  // accumulate-then-evict (se_h2o_accumulate_evict's rule) on h2o_pos / h2o_acc,
  // the slot that received the token being slot[unit] (or seq_len - 1), and
  // writes the evicted slot (or -1) to h2o_evict.
  int32_t* h2o_pos; float* h2o_acc; int32_t* h2o_evict; int h2o_cur, h2o_heavy, h2o_recent, h2o;
};
constexpr int ATTN_H2O_LDS_LOGITS = 12288;   // G * capacity logits held in LDS by the H2O step
constexpr int ATTN_H2O_SLOTS_PER_THREAD = 8;   // capacity <= 256 * this

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

// ------------------------------------------------------------------ split-K completion
// Every block of a split-K launch stores its partial (max, sum, output) and then
// takes a ticket on its (unit, head group) counter (block_ticket_last); the
// block that takes the last ticket merges all partials by log-sum-exp and
// resets the counter, so the workspace is zero again when the launch ends.
// Partial store: a device-scope write-through store when the launch merges in-kernel,
// a plain store when the combine kernel (a later launch) reads it.
__device__ __forceinline__ void st_part(const AttnArgs& a, float* p, float v) {
  if (a.fused) st_dev(p, v); else *p = v;
}

__device__ __forceinline__ bool attn_split_done(int* ctr, int splits) { return block_ticket_last(ctr, splits); }

// Merge the splits of heads [h0, h0 + nh) of one unit into out / lse (natural-log
// lse) and reset the unit's ticket counter.  A thread owns four consecutive
// output columns of one head; for a batch of up to SU splits it issues every
// load (max and sum as one 8-byte access, the four partial outputs as two)
// before using any, and folds the batch into a running (max, sum, output) by
// log-sum-exp, so a merge of up to SU splits costs one round trip.
template <int NT, int SU>
__device__ void attn_merge_splits_su(const AttnArgs& a, int unit, int h0, int nh, int* ctr) {
  const int S = a.splits, G = a.G, Dv = a.Dv;   // Dv is a multiple of 8
  const int b = unit / a.Hkv, kvh = unit % a.Hkv;
  const float* pml = a.part_ml + size_t(unit) * S * G * 2;
  const float* po = a.part_o + size_t(unit) * S * G * Dv;
  const size_t row0 = size_t(b) * a.Hq + size_t(kvh) * G + h0;
  for (int e = threadIdx.x * 4; e < nh * Dv; e += NT * 4) {
    const int hl = e / Dv, d0 = e - hl * Dv, h = h0 + hl;
    float M = -INFINITY, L = 0.f, O[4] = {0.f, 0.f, 0.f, 0.f};
    for (int s0 = 0; s0 < S; s0 += SU) {
      float2 mlb[SU], ob0[SU], ob1[SU];
#pragma unroll
      for (int j = 0; j < SU; ++j) {
        const int s = min(s0 + j, S - 1);
        mlb[j] = ld_dev2(pml + (s * G + h) * 2);
        const float* op = po + (size_t(s) * G + h) * Dv + d0;
        ob0[j] = ld_dev2(op);
        ob1[j] = ld_dev2(op + 2);
      }
      float Mb = -INFINITY;
#pragma unroll
      for (int j = 0; j < SU; ++j) {
        if (s0 + j >= S) mlb[j].x = -INFINITY;   // a repeated split, not counted
        Mb = fmaxf(Mb, mlb[j].x);
      }
      const float Mn = fmaxf(M, Mb);
      if (Mn == -INFINITY) continue;
      const float alpha = M == -INFINITY ? 0.f : ex2((M - Mn) * LOG2E);
      L *= alpha;
#pragma unroll
      for (int u = 0; u < 4; ++u) O[u] *= alpha;
#pragma unroll
      for (int j = 0; j < SU; ++j) {
        const float f = mlb[j].x == -INFINITY ? 0.f : ex2((mlb[j].x - Mn) * LOG2E);
        L += f * mlb[j].y;
        O[0] += f * ob0[j].x;
        O[1] += f * ob0[j].y;
        O[2] += f * ob1[j].x;
        O[3] += f * ob1[j].y;
      }
      M = Mn;
    }
    const float inv = L > 0.f ? 1.f / L : 0.f;
    *reinterpret_cast<float4*>(a.out + (row0 + hl) * Dv + d0) = make_float4(O[0] * inv, O[1] * inv, O[2] * inv, O[3] * inv);
    if (d0 == 0 && a.lse != nullptr) a.lse[row0 + hl] = L > 0.f ? M + logf(L) : -INFINITY;
  }
  if (threadIdx.x == 0) ticket_reset(ctr);
}

template <int NT>
__device__ void attn_merge_splits(const AttnArgs& a, int unit, int h0, int nh, int* ctr) {
  if (a.splits <= 4) attn_merge_splits_su<NT, 4>(a, unit, h0, nh, ctr);
  else attn_merge_splits_su<NT, 8>(a, unit, h0, nh, ctr);
}

// Final output of a unit handled by one block (splits == 1): out = O / L, lse = M + log L.
__device__ __forceinline__ void attn_write_final(const AttnArgs& a, size_t row, int d, float M, float L, float O) {
  a.out[row * a.Dv + d] = L > 0.f ? O * (1.f / L) : 0.f;
  if (d == 0 && a.lse != nullptr) a.lse[row] = L > 0.f ? M + logf(L) : -INFINITY;
}

bool attn_mfma_supported(const AttnArgs& a);
bool attn_mla_supported(const AttnArgs& a);
int attn_mla_auto_splits(int units, int G, int slots);
se_status launch_attn_mla(const AttnArgs& a, hipStream_t s);
int attn_mfma_auto_splits(int units, int slots);
se_status launch_attn_mfma(const AttnArgs& a, hipStream_t s);
int attn_mfma_sel_keys(int ncp);
int attn_mla_sel_keys(int ncp);

inline bool attn_mfma_eligible(const se_cache& c) {
  return c.dtype == SE_BF16 && !c.latent && (c.d_k == 128 || c.d_k == 64) && c.d_v == c.d_k &&
         c.n_q_heads / c.n_kv_heads <= 16;
}

inline bool attn_mla_eligible(const se_cache& c) {
  return c.dtype == SE_BF16 && c.latent && c.d_k == 576 && c.d_v == 512 && c.n_q_heads / c.n_kv_heads <= 64;
}

}  // namespace se
