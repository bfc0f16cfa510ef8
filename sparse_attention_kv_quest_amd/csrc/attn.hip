// Split-K flash decode over an AttentionView: the vector-ALU kernel (any
// element type, key width <= 576, value width <= 512, group <= 64), the
// workspace layout and the dispatch.  The bf16 MFMA paths live in
// attn_mfma.hip (GQA) and attn_mla.hip (576-wide latent rows); every kernel
// merges its own splits (the block finishing a unit's last split does it).
//
// tokendh.com explainer, section "把边界划在'生命周期'上", and the ai-feeds
// digest, section 方法 / 关键模块: every method's kept positions reach attention
// through one view format, so one kernel serves all of them.  A view entry
// names `gran` consecutive cache slots; slots past seq_len are skipped.
#include "se_internal.hpp"
#include "attn_common.hpp"

namespace se {

constexpr int VT = 16;  // slots per tile in the vector kernel

template <typename T, int MAXR>
__global__ __launch_bounds__(256) void attn_vector_kernel(AttnArgs a) {
  extern __shared__ float smem[];
  const int G = a.G, Dk = a.Dk, Dv = a.Dv;
  float* qs = smem;                    // [G][Dk]
  float* kt = qs + G * Dk;             // [VT][Dk]
  float* vt = kt + VT * Dk;            // [VT][Dv] (unused for latent caches)
  float* pt = vt + (a.latent ? 0 : VT * Dv);  // [G][VT]
  float* ms = pt + G * VT;             // [G] running max
  float* ls = ms + G;                  // [G] running sum
  float* al = ls + G;                  // [G] rescale of this tile
  int* tok = (int*)(al + G);           // [VT]

  const int unit = blockIdx.y, split = blockIdx.x;
  const int b = unit / a.Hkv, kvh = unit % a.Hkv;
  const int n_slots = view_slot_count(a, unit, b);
  const int chunk = (n_slots + a.splits - 1) / a.splits;
  const int s0 = min(n_slots, split * chunk), s1 = min(n_slots, s0 + chunk);

  const T* qg = (const T*)a.q + (size_t(b) * a.Hq + size_t(kvh) * G) * Dk;
  for (int i = threadIdx.x; i < G * Dk; i += 256) qs[i] = to_f32(qg[i]);
  for (int h = threadIdx.x; h < G; h += 256) { ms[h] = -INFINITY; ls[h] = 0.f; }
  const int R = (G * Dv + 255) / 256;
  float acc[MAXR];
#pragma unroll
  for (int r = 0; r < MAXR; ++r) acc[r] = 0.f;
  const T* ku = (const T*)a.k + size_t(unit) * a.cap * a.k_stride;
  const T* vu = a.latent ? ku : (const T*)a.v + size_t(unit) * a.cap * a.v_stride;
  const int vstride = a.latent ? a.k_stride : a.v_stride;
  __syncthreads();

  for (int t0 = s0; t0 < s1; t0 += VT) {
    const int nt = min(VT, s1 - t0);
    if (threadIdx.x < VT) tok[threadIdx.x] = threadIdx.x < nt ? view_token(a, unit, b, t0 + threadIdx.x) : -1;
    __syncthreads();
    for (int i = threadIdx.x; i < VT * Dk; i += 256) {
      const int j = i / Dk, d = i % Dk, t = tok[j];
      kt[i] = t >= 0 ? to_f32(ku[size_t(t) * a.k_stride + d]) : 0.f;
    }
    if (!a.latent)
      for (int i = threadIdx.x; i < VT * Dv; i += 256) {
        const int j = i / Dv, d = i % Dv, t = tok[j];
        vt[i] = t >= 0 ? to_f32(vu[size_t(t) * vstride + d]) : 0.f;
      }
    __syncthreads();
    // logits of (slot j, head h)
    for (int i = threadIdx.x; i < G * VT; i += 256) {
      const int h = i / VT, j = i % VT;
      float lg = -INFINITY;
      if (tok[j] >= 0) {
        float dot = 0.f;
        for (int d = 0; d < Dk; ++d) dot += qs[h * Dk + d] * kt[j * Dk + d];
        lg = dot * a.scale;
      }
      if (a.logits != nullptr && j < nt && t0 + j < a.logit_cap)
        a.logits[(size_t(b) * a.Hq + size_t(kvh) * G + h) * a.logit_cap + t0 + j] = lg;
      pt[i] = lg;
    }
    __syncthreads();
    // online softmax bookkeeping, one thread per head
    for (int h = threadIdx.x; h < G; h += 256) {
      float mt = -INFINITY;
      for (int j = 0; j < VT; ++j) mt = fmaxf(mt, pt[h * VT + j]);
      const float mo = ms[h], mn = fmaxf(mo, mt);
      float alpha = 1.f, sum = 0.f;
      if (mn != -INFINITY) {
        alpha = ex2((mo - mn) * LOG2E);
        for (int j = 0; j < VT; ++j) {
          float p = ex2((pt[h * VT + j] - mn) * LOG2E);
          pt[h * VT + j] = p;
          sum += p;
        }
      } else {
        for (int j = 0; j < VT; ++j) pt[h * VT + j] = 0.f;
      }
      ms[h] = mn;
      ls[h] = ls[h] * alpha + sum;
      al[h] = alpha;
    }
    __syncthreads();
    const float* vsrc = a.latent ? kt : vt;
    const int vs = a.latent ? Dk : Dv;
#pragma unroll
    for (int r = 0; r < MAXR; ++r) {
      const int pair = threadIdx.x + 256 * r;
      if (r < R && pair < G * Dv) {
        const int h = pair / Dv, d = pair % Dv;
        float o = acc[r] * al[h];
        for (int j = 0; j < VT; ++j) o += pt[h * VT + j] * vsrc[j * vs + d];
        acc[r] = o;
      }
    }
    __syncthreads();
  }
  if (a.splits == 1) {
    const size_t row0 = size_t(b) * a.Hq + size_t(kvh) * G;
#pragma unroll
    for (int r = 0; r < MAXR; ++r) {
      const int pair = threadIdx.x + 256 * r;
      if (r < R && pair < G * Dv) attn_write_final(a, row0 + pair / Dv, pair % Dv, ms[pair / Dv], ls[pair / Dv], acc[r]);
    }
    return;
  }
  // partial results of this split; the block finishing the unit's last split merges them
  float* pml = a.part_ml + (size_t(unit) * a.splits + split) * G * 2;
  float* po = a.part_o + (size_t(unit) * a.splits + split) * G * Dv;
  for (int h = threadIdx.x; h < G; h += 256) { st_part(a, pml + 2 * h, ms[h]); st_part(a, pml + 2 * h + 1, ls[h]); }
#pragma unroll
  for (int r = 0; r < MAXR; ++r) {
    const int pair = threadIdx.x + 256 * r;
    if (r < R && pair < G * Dv) st_part(a, po + pair, acc[r]);
  }
  if (!a.fused) return;
  int* ctr = a.counters + unit * ATTN_MAX_HG;
  if (attn_split_done(ctr, a.splits)) attn_merge_splits<256>(a, unit, 0, G, ctr);
}

// One block per (head of the group, unit): merge the split partials by log-sum-exp
// (used when a unit's partials are too large for one block to merge them quickly).
// The per-split weights exp(m_s - M) are formed once in LDS; the output pass then
// streams the partial outputs with independent loads.
__global__ __launch_bounds__(128) void attn_combine_kernel(AttnArgs a) {
  __shared__ float f_s[ATTN_MAX_SPLITS];
  __shared__ float red[2];
  const int unit = blockIdx.y, h = blockIdx.x;
  const int G = a.G, Dv = a.Dv, S = a.splits;
  const int b = unit / a.Hkv, kvh = unit % a.Hkv;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const float* pml = a.part_ml + size_t(unit) * S * G * 2;
  const float* po = a.part_o + size_t(unit) * S * G * Dv;
  const size_t row = size_t(b) * a.Hq + size_t(kvh) * G + h;
  constexpr int CS = 8, CD = 4;
  if (S <= CS && Dv == CD * 128) {
    // every load of the block at once (clamped split index, weight 0 past S): the
    // partial outputs, then each split's (max, sum), one round trip in all
    float pv[CS][CD];
#pragma unroll
    for (int sx = 0; sx < CS; ++sx)
#pragma unroll
      for (int j = 0; j < CD; ++j) pv[sx][j] = po[(size_t(min(sx, S - 1)) * G + h) * Dv + threadIdx.x + 128 * j];
    float2 ml[CS];
#pragma unroll
    for (int sx = 0; sx < CS; ++sx) ml[sx] = *reinterpret_cast<const float2*>(pml + (min(sx, S - 1) * G + h) * 2);
    float M = -INFINITY;
#pragma unroll
    for (int sx = 0; sx < CS; ++sx)
      if (sx < S) M = fmaxf(M, ml[sx].x);
    float f[CS], L = 0.f;
#pragma unroll
    for (int sx = 0; sx < CS; ++sx) {
      f[sx] = (sx < S && ml[sx].x != -INFINITY) ? ex2((ml[sx].x - M) * LOG2E) : 0.f;
      L += f[sx] * ml[sx].y;
    }
    const float inv = L > 0.f ? 1.f / L : 0.f;
#pragma unroll
    for (int j = 0; j < CD; ++j) {
      float o = 0.f;
#pragma unroll
      for (int sx = 0; sx < CS; ++sx) o += f[sx] * pv[sx][j];
      a.out[row * Dv + threadIdx.x + 128 * j] = o * inv;
    }
    if (threadIdx.x == 0 && a.lse != nullptr) a.lse[row] = L > 0.f ? M + logf(L) : -INFINITY;
    return;
  }
  float mloc = -INFINITY;
  for (int s = threadIdx.x; s < S; s += 128) {
    const float ms = pml[(s * G + h) * 2];
    f_s[s] = ms;
    mloc = fmaxf(mloc, ms);
  }
  mloc = wave_max(mloc);
  if (lane == 0) red[w] = mloc;
  __syncthreads();
  const float M = fmaxf(red[0], red[1]);
  __syncthreads();
  float lloc = 0.f;
  for (int s = threadIdx.x; s < S; s += 128) {
    const float ms = f_s[s];
    const float f = (ms != -INFINITY) ? ex2((ms - M) * LOG2E) : 0.f;
    f_s[s] = f;
    lloc += f * pml[(s * G + h) * 2 + 1];
  }
  lloc = wave_sum(lloc);
  if (lane == 0) red[w] = lloc;
  __syncthreads();
  const float L = red[0] + red[1];
  const float inv = L > 0.f ? 1.f / L : 0.f;
  for (int d = threadIdx.x; d < Dv; d += 128) {
    float o = 0.f;
#pragma unroll 8
    for (int s = 0; s < S; ++s) o += f_s[s] * po[(size_t(s) * G + h) * Dv + d];
    a.out[row * Dv + d] = o * inv;
  }
  if (threadIdx.x == 0 && a.lse != nullptr) a.lse[row] = L > 0.f ? M + logf(L) : -INFINITY;
}

int attn_auto_splits(const se_cache& c, int slots) {
  const int units = c.batch * c.n_kv_heads;
  if (attn_mfma_eligible(c)) return attn_mfma_auto_splits(units, slots);
  if (attn_mla_eligible(c)) return attn_mla_auto_splits(units, c.n_q_heads / c.n_kv_heads, slots);
  int s = ceil_div(1024, units);
  s = std::max(1, std::min(s, ceil_div(slots, 64)));
  return std::min(s, ATTN_MAX_SPLITS);
}

// Workspace: ticket counters (zero between calls), then the split partials.
size_t attn_counter_bytes(const se_cache& c) {
  return (size_t(c.batch) * c.n_kv_heads * ATTN_MAX_HG * sizeof(int) + 255) / 256 * 256;
}

size_t attn_ws_bytes(const se_cache& c, int slots, int num_splits) {
  const int S = num_splits > 0 ? num_splits : attn_auto_splits(c, slots);
  const size_t units = size_t(c.batch) * c.n_kv_heads, G = c.n_q_heads / c.n_kv_heads;
  return attn_counter_bytes(c) + units * S * G * (2 + size_t(c.d_v)) * sizeof(float);
}

se_status launch_attn_vector(const AttnArgs& a, hipStream_t s) {
  const int units = a.B * a.Hkv;
  const size_t lds_main = (size_t(a.G) * a.Dk + VT * a.Dk + (a.latent ? 0 : VT * a.Dv) + a.G * VT + 3 * a.G) *
                             sizeof(float) + VT * sizeof(int);
  const size_t lds = lds_main;
  if (lds > 160 * 1024) return SE_ERR_UNSUPPORTED;
  const int R = (a.G * a.Dv + 255) / 256;
  dim3 grid(a.splits, units);
#define SE_LAUNCH_VEC(TT, RR)                                                                       \
  do {                                                                                            \
    if (lds > 64 * 1024)                                                                          \
      (void)hipFuncSetAttribute((const void*)attn_vector_kernel<TT, RR>,                          \
                          hipFuncAttributeMaxDynamicSharedMemorySize, int(lds));                  \
    hipLaunchKernelGGL((attn_vector_kernel<TT, RR>), grid, dim3(256), lds, s, a);                  \
  } while (0)
  if (a.dtype == SE_F32) {
    if (R <= 4) SE_LAUNCH_VEC(float, 4);
    else if (R <= 16) SE_LAUNCH_VEC(float, 16);
    else if (R <= 64) SE_LAUNCH_VEC(float, 64);
    else return SE_ERR_UNSUPPORTED;
  } else {
    if (R <= 4) SE_LAUNCH_VEC(bf16_t, 4);
    else if (R <= 16) SE_LAUNCH_VEC(bf16_t, 16);
    else if (R <= 64) SE_LAUNCH_VEC(bf16_t, 64);
    else return SE_ERR_UNSUPPORTED;
  }
#undef SE_LAUNCH_VEC
  return launch_status();
}

// Fused append + attention: per batch row a ticket counter, then the attention workspace.
static size_t attn_row_ctr_bytes(const se_cache& c) { return (size_t(c.batch) * sizeof(int) + 255) / 256 * 256; }

size_t attn_append_ws_bytes(const se_cache& c, int slots, int num_splits) {
  return attn_row_ctr_bytes(c) + attn_ws_bytes(c, slots, num_splits);
}

se_status launch_append_attn(const se_cache& c, const void* q, void* k, void* v, const void* k_new,
                             const void* v_new, const int32_t* slot, int32_t* seq_len, const int32_t* view_idx,
                             const int32_t* view_len, int view_cap, int granularity, float scale, float* out,
                             float* lse, float* logits, int logit_cap, int num_splits, void* ws, hipStream_t s) {
  void* aws = (char*)ws + attn_row_ctr_bytes(c);
  AttnArgs a = make_attn_args(c, q, k, v, seq_len, view_idx, view_len, view_cap, granularity, scale, out,
                              lse, logits, logit_cap);
  const int slots = view_idx ? view_cap * granularity : c.capacity;
  a.splits = num_splits > 0 ? num_splits : attn_auto_splits(c, slots);
  if (!attn_mfma_supported(a)) {   // other shapes: the two calls' kernels (the same results)
    se_status st = launch_kv_append(c, k, v, k_new, v_new, slot, seq_len, s);
    if (st != SE_OK) return st;
    return launch_attn(c, q, k, v, seq_len, view_idx, view_len, view_cap, granularity, scale, out, lse, logits,
                       logit_cap, num_splits, aws, s);
  }
  a.counters = (int*)aws;
  a.part_ml = (float*)((char*)aws + attn_counter_bytes(c));
  a.part_o = a.part_ml + size_t(a.B) * a.Hkv * a.splits * a.G * 2;
  a.fused = a.splits > 1 && size_t(a.splits) * std::min(a.G, 32) * a.Dv * sizeof(float) <= ATTN_FUSED_MERGE_BYTES;
  a.app = 1;
  a.k_new = k_new; a.v_new = v_new; a.k_w = k; a.v_w = v;
  a.slot = slot; a.seq_len_w = seq_len; a.row_ctr = (int*)ws;
  se_status st = launch_attn_mfma(a, s);
  if (st != SE_OK || a.splits == 1 || a.fused) return st;
  hipLaunchKernelGGL(attn_combine_kernel, dim3(a.G, a.B * a.Hkv), dim3(128), 0, s, a);
  return launch_status();
}

// The Quest decode step: [workspace of the append + scoring launch][attention
// workspace with its batch-row tickets][view scratch for shapes that run the
// separate calls].
static size_t r256(size_t x) { return (x + 255) / 256 * 256; }

size_t quest_step_ws_bytes(const se_cache& c, int page_size, int top_pages) {
  const size_t units = size_t(c.batch) * c.n_kv_heads;
  return r256(quest_append_ws_bytes(c, page_size)) + r256(attn_append_ws_bytes(c, top_pages * page_size, 0)) +
         r256(units * (size_t(top_pages) + 1) * sizeof(int32_t));
}

se_status launch_quest_step(const se_cache& c, const void* q, void* k, void* v, const void* k_new,
                            const void* v_new, int32_t* seq_len, void* kmin, void* kmax, int page_size,
                            int top_pages, float scale, float* out, float* lse, int32_t* view_idx,
                            int32_t* view_len, float* page_score, void* ws, hipStream_t s) {
  const int units = c.batch * c.n_kv_heads, G = c.n_q_heads / c.n_kv_heads;
  const int ncp = ceil_div(c.capacity, page_size);
  char* ws_sel = (char*)ws;
  char* ws_att = ws_sel + r256(quest_append_ws_bytes(c, page_size));
  char* ws_view = ws_att + r256(attn_append_ws_bytes(c, top_pages * page_size, 0));
  AttnArgs a = make_attn_args(c, q, k, v, seq_len, nullptr, nullptr, 0, 1, scale, out, lse, nullptr, 0);
  a.view_cap = top_pages;
  a.gran = page_size;
  a.gshift = -1;
  for (int sh = 0; sh < 31; ++sh)
    if ((1 << sh) == page_size) { a.gshift = sh; break; }
  // GQA: attn_mfma_kernel; latent rows: attn_mla_pf_kernel (groups of 17..32 heads)
  const bool gqa = c.dtype == SE_BF16 && !c.latent && (c.d_k == 128 || c.d_k == 64) && G <= 16 &&
                   attn_mfma_sel_keys(ncp) > 0 && top_pages <= 2048 && a.gshift >= 0 && attn_mfma_supported(a);
  const bool mla = c.dtype == SE_BF16 && c.latent && c.d_k == 576 && c.d_v == 512 && G > 16 && G <= 32 &&
                   attn_mla_sel_keys(ncp) > 0 && top_pages <= 1024 && a.gshift >= 0 && attn_mla_supported(a);
  const bool fused = gqa || mla;
  if (!fused) {   // other shapes: the append + selection call, then the attention call (same results)
    int32_t* vi = view_idx ? view_idx : (int32_t*)ws_view;
    int32_t* vl = view_len ? view_len : (int32_t*)ws_view + size_t(units) * top_pages;
    se_status st = launch_quest_append(c, q, k, v, k_new, v_new, seq_len, kmin, kmax, page_size, top_pages, vi, vl,
                                       page_score, ws_sel, s);
    if (st != SE_OK) return st;
    return launch_attn(c, q, k, v, seq_len, vi, vl, top_pages, page_size, scale, out, lse, nullptr, 0, 0,
                       ws_att + attn_row_ctr_bytes(c), s, nullptr, nullptr);
  }
  // launch 1: the new rows, the appended page's min / max and every page's score
  float* score = nullptr;
  se_status st = launch_quest_append_scores(c, q, k, v, k_new, v_new, seq_len, kmin, kmax, page_size, page_score,
                                            ws_sel, &score, s);
  if (st != SE_OK) return st;
  // launch 2: per unit the top pages, then the attention over them; the new length
  a.splits = attn_auto_splits(c, top_pages * page_size);
  void* aws = ws_att + attn_row_ctr_bytes(c);
  a.counters = (int*)aws;
  a.part_ml = (float*)((char*)aws + attn_counter_bytes(c));
  a.part_o = a.part_ml + size_t(a.B) * a.Hkv * a.splits * a.G * 2;
  a.fused = a.splits > 1 && size_t(a.splits) * std::min(a.G, 32) * a.Dv * sizeof(float) <= ATTN_FUSED_MERGE_BYTES;
  a.row_ctr = (int*)ws_att;
  a.seq_len_w = seq_len;
  a.sel = gqa ? attn_mfma_sel_keys(ncp) : attn_mla_sel_keys(ncp);
  a.sel_score = score;
  a.sel_ncp = ncp;
  a.sel_view = view_idx;
  a.sel_vlen = view_len;
  st = gqa ? launch_attn_mfma(a, s) : launch_attn_mla(a, s);
  if (st != SE_OK || a.splits == 1 || a.fused) return st;
  hipLaunchKernelGGL(attn_combine_kernel, dim3(a.G, a.B * a.Hkv), dim3(128), 0, s, a);
  return launch_status();
}

// The Quest decode step over FP8 rows, in the same two launches and workspace as
// launch_quest_step: launch 1 quantizes the new rows, folds the stored K values into
// the appended page's min / max and scores every page; launch 2 selects each unit's
// pages and attends over the FP8 rows; other shapes run the separate calls' kernels.
se_status launch_quest_step_fp8(const se_cache& c, const void* q, void* kq, void* vq, uint8_t* ks, uint8_t* vs,
                                const void* k_new, const void* v_new, int32_t* seq_len, void* kmin, void* kmax,
                                int page_size, int top_pages, float scale, float* out, float* lse, int32_t* view_idx,
                                int32_t* view_len, float* page_score, void* ws, hipStream_t s) {
  const int units = c.batch * c.n_kv_heads, G = c.n_q_heads / c.n_kv_heads;
  const int ncp = ceil_div(c.capacity, page_size);
  char* ws_sel = (char*)ws;
  char* ws_att = ws_sel + r256(quest_append_ws_bytes(c, page_size));
  char* ws_view = ws_att + r256(attn_append_ws_bytes(c, top_pages * page_size, 0));
  AttnArgs a = make_attn_args(c, q, kq, vq, seq_len, nullptr, nullptr, 0, 1, scale, out, lse, nullptr, 0);
  a.k_scale = ks;
  a.v_scale = vs;
  a.fp8 = true;
  a.view_cap = top_pages;
  a.gran = page_size;
  a.gshift = -1;
  for (int sh = 0; sh < 31; ++sh)
    if ((1 << sh) == page_size) { a.gshift = sh; break; }
  // the attention over FP8 rows runs on the MFMA kernel only, over power-of-two page
  // views: reject anything else before anything is written
  if (a.gshift < 0 || !attn_mfma_supported(a)) return SE_ERR_UNSUPPORTED;
  const bool fused = c.dtype == SE_BF16 && !c.latent && (c.d_k == 128 || c.d_k == 64) && G <= 16 &&
                     attn_mfma_sel_keys(ncp) > 0 && top_pages <= 2048 && a.gshift >= 0;
  if (!fused) {   // other shapes: the three calls' kernels (same results)
    int32_t* vi = view_idx ? view_idx : (int32_t*)ws_view;
    int32_t* vl = view_len ? view_len : (int32_t*)ws_view + size_t(units) * top_pages;
    se_status st = launch_fp8_append(c, kq, vq, ks, vs, k_new, v_new, seq_len, kmin, kmax, page_size, s);
    if (st != SE_OK) return st;
    const size_t ctr_bytes = r256(size_t(c.batch) * sizeof(int));
    st = launch_quest(c, q, kmin, kmax, seq_len, page_size, top_pages, vi, vl, page_score, ws_sel + ctr_bytes, s);
    if (st != SE_OK) return st;
    return launch_attn(c, q, kq, vq, seq_len, vi, vl, top_pages, page_size, scale, out, lse, nullptr, 0, 0,
                       ws_att + attn_row_ctr_bytes(c), s, ks, vs);
  }
  float* score = nullptr;
  se_status st = launch_quest_fp8_append_scores(c, q, kq, vq, ks, vs, k_new, v_new, seq_len, kmin, kmax, page_size,
                                                page_score, ws_sel, &score, s);
  if (st != SE_OK) return st;
  a.splits = attn_auto_splits(c, top_pages * page_size);
  void* aws = ws_att + attn_row_ctr_bytes(c);
  a.counters = (int*)aws;
  a.part_ml = (float*)((char*)aws + attn_counter_bytes(c));
  a.part_o = a.part_ml + size_t(a.B) * a.Hkv * a.splits * a.G * 2;
  a.fused = a.splits > 1 && size_t(a.splits) * std::min(a.G, 32) * a.Dv * sizeof(float) <= ATTN_FUSED_MERGE_BYTES;
  a.row_ctr = (int*)ws_att;
  a.seq_len_w = seq_len;
  a.sel = attn_mfma_sel_keys(ncp);
  a.sel_score = score;
  a.sel_ncp = ncp;
  a.sel_view = view_idx;
  a.sel_vlen = view_len;
  st = launch_attn_mfma(a, s);
  if (st != SE_OK || a.splits == 1 || a.fused) return st;
  hipLaunchKernelGGL(attn_combine_kernel, dim3(a.G, a.B * a.Hkv), dim3(128), 0, s, a);
  return launch_status();
}

// The H2O decode step: [the fused attention's batch-row tickets and counters][logits
// and lse scratch for shapes that run the separate kernels].
size_t h2o_step_ws_bytes(const se_cache& c) {
  const size_t rows = size_t(c.batch) * c.n_q_heads;
  return r256(attn_append_ws_bytes(c, c.capacity, 1)) + r256(rows * size_t(c.capacity) * sizeof(float)) +
         r256(rows * sizeof(float));
}

__global__ void copy_or_fill_i32_kernel(int32_t* __restrict__ dst, const int32_t* __restrict__ src, int n) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) dst[i] = src != nullptr ? src[i] : -1;
}

se_status launch_h2o_step(const se_cache& c, const void* q, void* k, void* v, const void* k_new, const void* v_new,
                          const int32_t* slot_in, int32_t* seq_len, int32_t* slot_pos, float* acc, int cur_pos,
                          int heavy, int recent, float scale, float* out, float* lse, int32_t* evict_out, void* ws,
                          hipStream_t s) {
  const int units = c.batch * c.n_kv_heads, G = c.n_q_heads / c.n_kv_heads;
  char* ws_att = (char*)ws;
  float* lg_ws = (float*)(ws_att + r256(attn_append_ws_bytes(c, c.capacity, 1)));
  float* lse_ws = (float*)((char*)lg_ws + r256(size_t(c.batch) * c.n_q_heads * c.capacity * sizeof(float)));
  float* lse_o = lse ? lse : lse_ws;
  AttnArgs a = make_attn_args(c, q, k, v, seq_len, nullptr, nullptr, 0, 1, scale, out, lse_o, nullptr, 0);
  const bool fused = attn_mfma_supported(a) && int64_t(G) * c.capacity <= ATTN_H2O_LDS_LOGITS &&
                     c.capacity <= 256 * ATTN_H2O_SLOTS_PER_THREAD;
  if (!fused) {   // other shapes: append, attention with logits, accumulate + evict (the same results)
    se_status st = launch_kv_append(c, k, v, k_new, v_new, slot_in, seq_len, s);
    if (st != SE_OK) return st;
    st = launch_attn(c, q, k, v, seq_len, nullptr, nullptr, 0, 1, scale, out, lse_o, lg_ws, c.capacity, 1,
                     ws_att + attn_row_ctr_bytes(c), s, nullptr, nullptr);
    if (st != SE_OK) return st;
    hipLaunchKernelGGL(copy_or_fill_i32_kernel, dim3(ceil_div(units, 256)), dim3(256), 0, s, evict_out, slot_in, units);
    if (hipGetLastError() != hipSuccess) return SE_ERR_HIP;
    return launch_h2o(c, lg_ws, lse_o, c.capacity, seq_len, slot_pos, acc, cur_pos, heavy, recent, evict_out, s);
  }
  a.splits = 1;
  a.counters = (int*)(ws_att + attn_row_ctr_bytes(c));
  a.part_ml = (float*)((char*)a.counters + attn_counter_bytes(c));
  a.part_o = a.part_ml + size_t(units) * G * 2;
  a.fused = 0;
  a.logit_cap = c.capacity;
  a.app = 1;
  a.k_new = k_new; a.v_new = v_new; a.k_w = k; a.v_w = v;
  a.slot = slot_in; a.seq_len_w = seq_len; a.row_ctr = (int*)ws_att;
  a.h2o = 1;
  a.h2o_pos = slot_pos; a.h2o_acc = acc; a.h2o_evict = evict_out;
  a.h2o_cur = cur_pos; a.h2o_heavy = heavy; a.h2o_recent = recent;
  return launch_attn_mfma(a, s);
}

se_status launch_attn(const se_cache& c, const void* q, const void* k, const void* v,
                      const int32_t* seq_len, const int32_t* view_idx, const int32_t* view_len,
                      int view_cap, int granularity, float scale, float* out, float* lse,
                      float* logits, int logit_cap, int num_splits, void* ws, hipStream_t s,
                      const uint8_t* k_scale, const uint8_t* v_scale) {
  AttnArgs a = make_attn_args(c, q, k, v, seq_len, view_idx, view_len, view_cap, granularity, scale, out,
                              lse, logits, logit_cap);
  a.k_scale = k_scale;
  a.v_scale = v_scale;
  a.fp8 = k_scale != nullptr;
  const int slots = view_idx ? view_cap * granularity : c.capacity;
  a.splits = num_splits > 0 ? num_splits : attn_auto_splits(c, slots);
  a.counters = (int*)ws;
  a.part_ml = (float*)((char*)ws + attn_counter_bytes(c));
  a.part_o = a.part_ml + size_t(a.B) * a.Hkv * a.splits * a.G * 2;
  // one block merges a unit's splits when their partials are small; large ones
  // (MLA: 32 heads x 512 columns per split) go to the combine kernel
  a.fused = a.splits > 1 && size_t(a.splits) * std::min(a.G, 32) * a.Dv * sizeof(float) <= ATTN_FUSED_MERGE_BYTES;
  se_status st = SE_ERR_UNSUPPORTED;
  if (a.fp8) {   // FP8 rows: the MFMA kernel only
    if (!attn_mfma_supported(a)) return SE_ERR_UNSUPPORTED;
    st = launch_attn_mfma(a, s);
  } else if (attn_mfma_supported(a)) st = launch_attn_mfma(a, s);
  else if (attn_mla_supported(a)) st = launch_attn_mla(a, s);
  if (st == SE_ERR_UNSUPPORTED) st = launch_attn_vector(a, s);
  if (st != SE_OK || a.splits == 1 || a.fused) return st;
  hipLaunchKernelGGL(attn_combine_kernel, dim3(a.G, a.B * a.Hkv), dim3(128), 0, s, a);
  return launch_status();
}

}  // namespace se
