// H2O accumulate-then-evict and OmniKV filter-layer top-k.
//
// tokendh.com explainer, section "历史太长,会撑爆什么": H2O keeps a running
// table of accumulated attention scores and physically deletes entries;
// section "把边界划在'生命周期'上": it updates the scores at every decode step
// and then picks what to delete, while OmniKV decides at some layers which
// history matters and lets the following layers reuse that decision.
// Both consume the logits and log-sum-exp of a full-view decode attention.
#include "se_internal.hpp"

namespace se {

// ------------------------------------------------------------------ H2O
// One block per unit.  See se_h2o_accumulate_evict for the contract.
__global__ __launch_bounds__(256) void h2o_kernel(
    const float* __restrict__ logits, const float* __restrict__ lse, int logit_cap,
    const int32_t* __restrict__ seq_len, int32_t* __restrict__ slot_pos, float* __restrict__ acc,
    int32_t* __restrict__ evict_slot, int Hkv, int G, int cap, int cur_pos, int heavy, int recent) {
  __shared__ float lse_s[64];
  __shared__ int cnt_s[4];
  __shared__ uint64_t key_s[4];
  const int unit = blockIdx.x, b = unit / Hkv, kvh = unit % Hkv;
  const int n = min(seq_len[b], cap);
  int32_t* pos = slot_pos + size_t(unit) * cap;
  float* a = acc + size_t(unit) * cap;
  const float* lg = logits + (size_t(b) * Hkv * G + size_t(kvh) * G) * logit_cap;
  for (int h = threadIdx.x; h < G; h += blockDim.x) lse_s[h] = lse[size_t(b) * Hkv * G + size_t(kvh) * G + h];
  if (threadIdx.x == 0) {
    const int in = evict_slot[unit];
    const int ns = in >= 0 ? in : n - 1;
    if (ns >= 0 && ns < cap) { pos[ns] = cur_pos; a[ns] = 0.f; }
  }
  __syncthreads();
  // accumulate: every occupied slot adds the group's softmax weight on it
  int cnt = 0;
  for (int s = threadIdx.x; s < n; s += blockDim.x) {
    if (pos[s] < 0) continue;
    float p = 0.f;
    for (int h = 0; h < G; ++h) {
      const float l = lse_s[h];
      if (l != -INFINITY) p += h2o_exp(lg[size_t(h) * logit_cap + s] - l);
    }
    a[s] += p;
    ++cnt;
  }
  // count occupied slots
  cnt = wave_sum_i(cnt);
  const int lane = threadIdx.x & (WAVE - 1), w = threadIdx.x / WAVE;
  if (lane == 0) cnt_s[w] = cnt;
  __syncthreads();
  const int occupied = cnt_s[0] + cnt_s[1] + cnt_s[2] + cnt_s[3];
  if (occupied <= heavy + recent) {
    if (threadIdx.x == 0) evict_slot[unit] = -1;
    return;
  }
  // argmin of (score, position) over slots outside the recent window
  uint64_t best = ~0ull;
  int best_slot = -1;
  for (int s = threadIdx.x; s < n; s += blockDim.x) {
    const int p = pos[s];
    if (p < 0 || p > cur_pos - recent) continue;
    const uint64_t key = (uint64_t(ordered_bits(a[s])) << 32) | uint64_t(uint32_t(p));
    if (key < best) { best = key; best_slot = s; }
  }
  for (int o = 32; o > 0; o >>= 1) {
    const uint64_t t = __shfl_xor(best, o, WAVE);
    const int ts = __shfl_xor(best_slot, o, WAVE);
    if (t < best) { best = t; best_slot = ts; }
  }
  __shared__ int slot_s[4];
  if (lane == 0) { key_s[w] = best; slot_s[w] = best_slot; }
  __syncthreads();
  if (threadIdx.x == 0) {
    uint64_t k = key_s[0];
    int ev = slot_s[0];
    for (int i = 1; i < 4; ++i)
      if (key_s[i] < k) { k = key_s[i]; ev = slot_s[i]; }
    if (ev >= 0) { pos[ev] = -1; a[ev] = 0.f; }
    evict_slot[unit] = ev;
  }
}

// Register-resident variant for capacities up to 256 * E: thread t holds
// slots t, t + 256, ... (coalesced), takes the new token's slot into its own
// registers, accumulates the group's softmax weights with all of its logit
// loads in flight, counts and finds the argmin of (score, position) with DPP
// reductions, and needs one block barrier per reduction.
__device__ __forceinline__ uint32_t wave_min_u32(uint32_t v) {
  return wave_last(wave_incl_scan_dpp(v, ~0u, [](uint32_t x, uint32_t y) { return x < y ? x : y; }));
}

template <int E>
__global__ __launch_bounds__(256) void h2o_reg_kernel(
    const float* __restrict__ logits, const float* __restrict__ lse, int logit_cap,
    const int32_t* __restrict__ seq_len, int32_t* __restrict__ slot_pos, float* __restrict__ acc,
    int32_t* __restrict__ evict_slot, int Hkv, int G, int cap, int cur_pos, int heavy, int recent) {
  __shared__ int cnt_s[4];
  __shared__ uint32_t hi_s[4], lo_s[4];
  __shared__ int slot_s[4];
  const int unit = blockIdx.x, b = unit / Hkv, kvh = unit % Hkv;
  const int lane = threadIdx.x & (WAVE - 1), w = threadIdx.x / WAVE;
  const int n = min(seq_len[b], cap);
  int32_t* pos = slot_pos + size_t(unit) * cap;
  float* a = acc + size_t(unit) * cap;
  const size_t row0 = size_t(b) * Hkv * G + size_t(kvh) * G;
  const float* lg = logits + row0 * logit_cap;
  const int in = evict_slot[unit];
  const int ns = in >= 0 ? in : n - 1;   // the slot that received the token at cur_pos
  if (threadIdx.x == 0 && ns >= n && ns < cap) { pos[ns] = cur_pos; a[ns] = 0.f; }   // outside the attended slots
  // the slot state and the first HC heads' logits go out together (unconditional
  // loads at clamped indices, masked after): one memory round trip before the
  // accumulation instead of two
  int p[E];
  float sc[E];
#pragma unroll
  for (int j = 0; j < E; ++j) {
    const int s = max(min(j * 256 + int(threadIdx.x), n - 1), 0);
    p[j] = pos[s];
    sc[j] = a[s];
  }
  // accumulate: every occupied slot adds the group's softmax weight on it, heads in
  // ascending order; the logit loads of HC heads go out together (one memory round
  // trip per HC heads, not per head)
  constexpr int HC = E <= 8 ? 8 : 4;
  auto load_heads = [&](int h0, float (&l)[HC], float (&x)[HC][E]) {
#pragma unroll
    for (int hh = 0; hh < HC; ++hh) {
      const int h = min(h0 + hh, G - 1);
      l[hh] = h0 + hh < G ? lse[row0 + h] : -INFINITY;
#pragma unroll
      for (int j = 0; j < E; ++j) x[hh][j] = lg[size_t(h) * logit_cap + min(j * 256 + int(threadIdx.x), logit_cap - 1)];
    }
  };
  auto add_heads = [&](const float (&l)[HC], const float (&x)[HC][E]) {
#pragma unroll
    for (int hh = 0; hh < HC; ++hh) {
      if (l[hh] == -INFINITY) continue;
#pragma unroll
      for (int j = 0; j < E; ++j)
        if (p[j] >= 0) sc[j] += h2o_exp(x[hh][j] - l[hh]);
    }
  };
  {
    float l[HC], x[HC][E];
    load_heads(0, l, x);
#pragma unroll
    for (int j = 0; j < E; ++j) {
      const int s = j * 256 + threadIdx.x;
      if (s >= n) { p[j] = -1; sc[j] = 0.f; }
      if (s == ns) { p[j] = cur_pos; sc[j] = 0.f; }
    }
    add_heads(l, x);
  }
  for (int h0 = HC; h0 < G; h0 += HC) {
    float l[HC], x[HC][E];
    load_heads(h0, l, x);
    add_heads(l, x);
  }
  int cnt = 0;
#pragma unroll
  for (int j = 0; j < E; ++j) {
    const int s = j * 256 + threadIdx.x;
    if (s < n) {
      if (s == ns) pos[s] = cur_pos;
      if (p[j] >= 0) a[s] = sc[j];
      else if (s == ns) a[s] = 0.f;
      cnt += p[j] >= 0;
    }
  }
  cnt = wave_sum_i(cnt);
  if (lane == 0) cnt_s[w] = cnt;
  __syncthreads();
  const int occupied = cnt_s[0] + cnt_s[1] + cnt_s[2] + cnt_s[3];
  if (occupied <= heavy + recent) {
    if (threadIdx.x == 0) evict_slot[unit] = -1;
    return;
  }
  // argmin of (score, position) over slots outside the recent window: the
  // ordered score bits first, then the position among the lanes that hold it
  uint32_t bh = ~0u, bl = ~0u;
  int bs = -1;
#pragma unroll
  for (int j = 0; j < E; ++j) {
    const int s = j * 256 + threadIdx.x;
    if (s < n && p[j] >= 0 && p[j] <= cur_pos - recent) {
      const uint32_t hkey = ordered_bits(sc[j]), lkey = uint32_t(p[j]);
      if (hkey < bh || (hkey == bh && lkey < bl)) { bh = hkey; bl = lkey; bs = s; }
    }
  }
  const uint32_t wh = wave_min_u32(bh);
  const uint32_t wl = wave_min_u32(bh == wh ? bl : ~0u);
  const uint64_t hit = __ballot(bh == wh && bl == wl && bs >= 0);
  const int ws = hit ? __builtin_amdgcn_readlane(bs, __ffsll((unsigned long long)hit) - 1) : -1;
  if (lane == 0) { hi_s[w] = wh; lo_s[w] = wl; slot_s[w] = ws; }
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t kh = hi_s[0], kl = lo_s[0];
    int ev = slot_s[0];
    for (int i = 1; i < 4; ++i)
      if (slot_s[i] >= 0 && (ev < 0 || hi_s[i] < kh || (hi_s[i] == kh && lo_s[i] < kl))) {
        kh = hi_s[i]; kl = lo_s[i]; ev = slot_s[i];
      }
    if (ev >= 0) { pos[ev] = -1; a[ev] = 0.f; }
    evict_slot[unit] = ev;
  }
}

se_status launch_h2o(const se_cache& c, const float* logits, const float* lse, int logit_cap,
                     const int32_t* seq_len, int32_t* slot_pos, float* acc, int cur_pos, int heavy,
                     int recent, int32_t* evict_slot, hipStream_t s) {
  const int G = c.n_q_heads / c.n_kv_heads;
  const dim3 grid(c.batch * c.n_kv_heads);
#define SE_H2O(KERN) hipLaunchKernelGGL(KERN, grid, dim3(256), 0, s, logits, lse, logit_cap, seq_len, slot_pos, acc, \
                                        evict_slot, c.n_kv_heads, G, c.capacity, cur_pos, heavy, recent)
  if (c.capacity <= 256 * 2) SE_H2O(h2o_reg_kernel<2>);
  else if (c.capacity <= 256 * 4) SE_H2O(h2o_reg_kernel<4>);
  else if (c.capacity <= 256 * 8) SE_H2O(h2o_reg_kernel<8>);
  else if (c.capacity <= 256 * 16) SE_H2O(h2o_reg_kernel<16>);
  else SE_H2O(h2o_kernel);
#undef SE_H2O
  return launch_status();
}

// ------------------------------------------------------------------ OmniKV
// Two launches: a score pass over every (unit, slot) with all of a thread's
// logit loads in flight, then one block per unit selects the top_k slots.
constexpr int OMNI_BLOCK = 1024;
constexpr int OMNI_SPT = 4;   // slots per thread of the score pass

// grid (slot groups of 1024, units): score[j] = sum over the group's heads of exp(logit_hj - lse_h).
__global__ __launch_bounds__(256) void omnikv_score_kernel(const float* __restrict__ logits,
                                                           const float* __restrict__ lse, int logit_cap,
                                                           const int32_t* __restrict__ seq_len,
                                                           float* __restrict__ score, int Hkv, int G) {
  const int unit = blockIdx.y, b = unit / Hkv, kvh = unit % Hkv;
  const int n = min(seq_len[b], logit_cap);
  const size_t row0 = size_t(b) * Hkv * G + size_t(kvh) * G;
  const float* lg = logits + row0 * logit_cap;
  const int j0 = blockIdx.x * 256 * OMNI_SPT + threadIdx.x;
  float p[OMNI_SPT] = {};
  // heads in ascending order; the logit loads of 8 heads go out together
  constexpr int HC = 8;
  for (int h0 = 0; h0 < G; h0 += HC) {
    float l[HC], x[HC][OMNI_SPT];
#pragma unroll
    for (int hh = 0; hh < HC; ++hh) {
      const int h = min(h0 + hh, G - 1);
      l[hh] = h0 + hh < G ? lse[row0 + h] : -INFINITY;
#pragma unroll
      for (int u = 0; u < OMNI_SPT; ++u) x[hh][u] = lg[size_t(h) * logit_cap + min(j0 + 256 * u, logit_cap - 1)];
    }
#pragma unroll
    for (int hh = 0; hh < HC; ++hh) {
      if (l[hh] == -INFINITY) continue;
#pragma unroll
      for (int u = 0; u < OMNI_SPT; ++u) p[u] += expf(x[hh][u] - l[hh]);
    }
  }
#pragma unroll
  for (int u = 0; u < OMNI_SPT; ++u)
    if (j0 + 256 * u < n) score[size_t(unit) * logit_cap + j0 + 256 * u] = p[u];
}

template <int E>
__global__ __launch_bounds__(OMNI_BLOCK) void omnikv_topk_reg_kernel(const float* __restrict__ score, int logit_cap,
                                                                     const int32_t* __restrict__ seq_len,
                                                                     int32_t* __restrict__ view_idx,
                                                                     int32_t* __restrict__ view_len, int Hkv,
                                                                     int top_k) {
  __shared__ TopkRegShared sh;
  const int unit = blockIdx.x, b = unit / Hkv;
  const int n = min(seq_len[b], logit_cap);
  const float* su = score + size_t(unit) * logit_cap;
  const int kk = block_topk_reg<OMNI_BLOCK, E>([&](int j) { return su[j]; }, n, top_k,
                                               view_idx + size_t(unit) * top_k, sh);
  if (threadIdx.x == 0) view_len[unit] = kk;
}

// Longer caches: the LDS / global-memory block top-k over the stored scores.
__global__ __launch_bounds__(OMNI_BLOCK) void omnikv_topk_block_kernel(const float* __restrict__ score,
                                                                       int logit_cap,
                                                                       const int32_t* __restrict__ seq_len,
                                                                       int32_t* __restrict__ view_idx,
                                                                       int32_t* __restrict__ view_len, int Hkv,
                                                                       int top_k) {
  __shared__ TopkShared sh;
  const int unit = blockIdx.x, b = unit / Hkv;
  const int n = min(seq_len[b], logit_cap);
  const float* su = score + size_t(unit) * logit_cap;
  const int kk = block_topk_ascending<OMNI_BLOCK>([&](int i) { return su[i]; }, n, top_k,
                                                  view_idx + size_t(unit) * top_k, sh);
  if (threadIdx.x == 0) view_len[unit] = kk;
}

size_t omnikv_ws_bytes(const se_cache& c, int logit_cap, int /*top_k*/) {
  return size_t(c.batch) * c.n_kv_heads * logit_cap * sizeof(float);
}

se_status launch_omnikv(const se_cache& c, const float* logits, const float* lse, int logit_cap,
                        const int32_t* seq_len, int top_k, int32_t* view_idx, int32_t* view_len,
                        float* scores, void* ws, hipStream_t s) {
  const int G = c.n_q_heads / c.n_kv_heads, units = c.batch * c.n_kv_heads;
  float* sc = scores ? scores : (float*)ws;
  hipLaunchKernelGGL(omnikv_score_kernel, dim3(ceil_div(logit_cap, 256 * OMNI_SPT), units), dim3(256), 0, s, logits,
                     lse, logit_cap, seq_len, sc, c.n_kv_heads, G);
#define SE_OMNI(KERN) hipLaunchKernelGGL(KERN, dim3(units), dim3(OMNI_BLOCK), 0, s, sc, logit_cap, seq_len, view_idx, \
                                         view_len, c.n_kv_heads, top_k)
  if (logit_cap <= OMNI_BLOCK * 8) SE_OMNI(omnikv_topk_reg_kernel<8>);
  else if (logit_cap <= OMNI_BLOCK * 16) SE_OMNI(omnikv_topk_reg_kernel<16>);
  else if (logit_cap <= OMNI_BLOCK * 24) SE_OMNI(omnikv_topk_reg_kernel<24>);
  else SE_OMNI(omnikv_topk_block_kernel);
#undef SE_OMNI
  return launch_status();
}

}  // namespace se
