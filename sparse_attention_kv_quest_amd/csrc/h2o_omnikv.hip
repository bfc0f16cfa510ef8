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
      if (l != -INFINITY) p += expf(lg[size_t(h) * logit_cap + s] - l);
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

se_status launch_h2o(const se_cache& c, const float* logits, const float* lse, int logit_cap,
                     const int32_t* seq_len, int32_t* slot_pos, float* acc, int cur_pos, int heavy,
                     int recent, int32_t* evict_slot, hipStream_t s) {
  const int G = c.n_q_heads / c.n_kv_heads;
  hipLaunchKernelGGL(h2o_kernel, dim3(c.batch * c.n_kv_heads), dim3(256), 0, s, logits, lse, logit_cap,
                     seq_len, slot_pos, acc, evict_slot, c.n_kv_heads, G, c.capacity, cur_pos, heavy, recent);
  return launch_status();
}

// ------------------------------------------------------------------ OmniKV
constexpr int OMNI_BLOCK = 1024;
constexpr int OMNI_LDS = 32768;  // scores kept in LDS up to this many slots (128 KiB)

template <bool IN_LDS>
__global__ __launch_bounds__(OMNI_BLOCK) void omnikv_kernel(
    const float* __restrict__ logits, const float* __restrict__ lse, int logit_cap,
    const int32_t* __restrict__ seq_len, int32_t* __restrict__ view_idx, int32_t* __restrict__ view_len,
    float* __restrict__ scores_out, float* __restrict__ ws, int Hkv, int G, int top_k) {
  extern __shared__ float s_lds[];
  __shared__ TopkShared sh;
  __shared__ float lse_s[64];
  const int unit = blockIdx.x, b = unit / Hkv, kvh = unit % Hkv;
  const int n = min(seq_len[b], logit_cap);
  const float* lg = logits + (size_t(b) * Hkv * G + size_t(kvh) * G) * logit_cap;
  float* sc = IN_LDS ? s_lds : ws + size_t(unit) * logit_cap;
  for (int h = threadIdx.x; h < G; h += OMNI_BLOCK) lse_s[h] = lse[size_t(b) * Hkv * G + size_t(kvh) * G + h];
  __syncthreads();
  for (int j = threadIdx.x; j < n; j += OMNI_BLOCK) {
    float p = 0.f;
    for (int h = 0; h < G; ++h) {
      const float l = lse_s[h];
      if (l != -INFINITY) p += expf(lg[size_t(h) * logit_cap + j] - l);
    }
    sc[j] = p;
    if (scores_out) scores_out[size_t(unit) * logit_cap + j] = p;
  }
  __syncthreads();
  const int kk = block_topk_ascending<OMNI_BLOCK>([&](int i) { return sc[i]; }, n, top_k,
                                                  view_idx + size_t(unit) * top_k, sh);
  if (threadIdx.x == 0) view_len[unit] = kk;
}

size_t omnikv_ws_bytes(const se_cache& c, int logit_cap, int /*top_k*/) {
  return logit_cap <= OMNI_LDS ? 0 : size_t(c.batch) * c.n_kv_heads * logit_cap * sizeof(float);
}

se_status launch_omnikv(const se_cache& c, const float* logits, const float* lse, int logit_cap,
                        const int32_t* seq_len, int top_k, int32_t* view_idx, int32_t* view_len,
                        float* scores, void* ws, hipStream_t s) {
  const int G = c.n_q_heads / c.n_kv_heads, units = c.batch * c.n_kv_heads;
  if (logit_cap <= OMNI_LDS) {
    const size_t lds = size_t(logit_cap) * sizeof(float);
    (void)hipFuncSetAttribute((const void*)omnikv_kernel<true>, hipFuncAttributeMaxDynamicSharedMemorySize,
                        int(OMNI_LDS * sizeof(float)));
    hipLaunchKernelGGL(omnikv_kernel<true>, dim3(units), dim3(OMNI_BLOCK), lds, s, logits, lse, logit_cap,
                       seq_len, view_idx, view_len, scores, (float*)nullptr, c.n_kv_heads, G, top_k);
  } else {
    hipLaunchKernelGGL(omnikv_kernel<false>, dim3(units), dim3(OMNI_BLOCK), 0, s, logits, lse, logit_cap,
                       seq_len, view_idx, view_len, scores, (float*)ws, c.n_kv_heads, G, top_k);
  }
  return launch_status();
}

}  // namespace se
