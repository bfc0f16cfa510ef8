// Quest page scoring and top-k page view.
//
// tokendh.com explainer, section "历史太长,会撑爆什么": Quest chooses pages per
// query from a summary index kept beside the full history.  A page's score for
// query head h is the upper bound sum_d max(q_hd * min_pd, q_hd * max_pd) of
// q_h . k over the page, i.e. sum_d (q+_hd * max_pd + q-_hd * min_pd) with
// q+ = max(q, 0), q- = min(q, 0); a KV head's page score is the max over the
// heads of its group.  The view is the top pages (ties to the lower page),
// in ascending page order.
#include "se_internal.hpp"

namespace se {

constexpr int QUEST_TOPK_LDS = 8192;  // page scores held in LDS by the top-k kernel

// ------------------------------------------------------------------ vector scoring (any dtype / width)
// grid: (page blocks, units); block 256 threads = PPB pages x G heads (G <= 64).
// q of the group is staged in LDS as fp32 split into q+ and q-.
template <typename T>
__global__ __launch_bounds__(256) void quest_score_vector_kernel(
    const T* __restrict__ q, const T* __restrict__ kmin, const T* __restrict__ kmax,
    const int32_t* __restrict__ seq_len, float* __restrict__ score, int Hkv, int G, int D, int P,
    int n_cap_pages) {
  extern __shared__ float smem[];
  float* qp = smem;            // [G][D]
  float* qn = smem + G * D;    // [G][D]
  float* ub = qn + G * D;      // [256]
  const int unit = blockIdx.y, b = unit / Hkv, kvh = unit % Hkv;
  const int npages = min((seq_len[b] + P - 1) / P, n_cap_pages);
  const T* qg = q + (size_t(b) * Hkv * G + size_t(kvh) * G) * D;
  for (int i = threadIdx.x; i < G * D; i += blockDim.x) {
    float x = to_f32(qg[i]);
    qp[i] = fmaxf(x, 0.f);
    qn[i] = fminf(x, 0.f);
  }
  __syncthreads();
  const int ppb = blockDim.x / G;
  const int lp = threadIdx.x / G, h = threadIdx.x % G;
  const int p = blockIdx.x * ppb + lp;
  float u = -INFINITY;
  if (lp < ppb && p < npages) {
    const T* mn = kmin + (size_t(unit) * n_cap_pages + p) * D;
    const T* mx = kmax + (size_t(unit) * n_cap_pages + p) * D;
    float acc = 0.f;
    for (int d = 0; d < D; ++d) acc += qp[h * D + d] * to_f32(mx[d]) + qn[h * D + d] * to_f32(mn[d]);
    u = acc;
  }
  ub[threadIdx.x] = u;
  __syncthreads();
  if (threadIdx.x < ppb) {
    const int pp = blockIdx.x * ppb + threadIdx.x;
    if (pp < n_cap_pages) {
      float s = -INFINITY;
      for (int j = 0; j < G; ++j) s = fmaxf(s, ub[threadIdx.x * G + j]);
      score[size_t(unit) * n_cap_pages + pp] = pp < npages ? s : -INFINITY;
    }
  }
}

// ------------------------------------------------------------------ top-k pages
// One block per unit: page scores -> ascending view of the best top_pages valid pages.
template <int BLOCK>
__global__ __launch_bounds__(BLOCK) void quest_topk_kernel(
    const float* __restrict__ score, const int32_t* __restrict__ seq_len, int32_t* __restrict__ view_idx,
    int32_t* __restrict__ view_len, int Hkv, int P, int n_cap_pages, int top_pages) {
  __shared__ float s_lds[QUEST_TOPK_LDS];
  __shared__ TopkShared sh;
  const int unit = blockIdx.x, b = unit / Hkv;
  const int n = min((seq_len[b] + P - 1) / P, n_cap_pages);
  const float* su = score + size_t(unit) * n_cap_pages;
  int32_t* out = view_idx + size_t(unit) * top_pages;
  int kk;
  if (n <= QUEST_TOPK_LDS) {
    for (int i = threadIdx.x; i < n; i += BLOCK) s_lds[i] = su[i];
    __syncthreads();
    kk = block_topk_ascending<BLOCK>([&](int i) { return s_lds[i]; }, n, top_pages, out, sh);
  } else {
    kk = block_topk_ascending<BLOCK>([&](int i) { return su[i]; }, n, top_pages, out, sh);
  }
  if (threadIdx.x == 0) view_len[unit] = kk;
}

size_t quest_ws_bytes(const se_cache& c, int page_size, int /*top_pages*/) {
  return size_t(c.batch) * c.n_kv_heads * ceil_div(c.capacity, page_size) * sizeof(float);
}

se_status launch_quest(const se_cache& c, const void* q, const void* kmin, const void* kmax,
                       const int32_t* seq_len, int page_size, int top_pages, int32_t* view_idx,
                       int32_t* view_len, float* page_score, void* ws, hipStream_t s) {
  const int units = c.batch * c.n_kv_heads, G = c.n_q_heads / c.n_kv_heads;
  const int ncp = ceil_div(c.capacity, page_size);
  float* score = page_score ? page_score : (float*)ws;
  const int ppb = 256 / G;
  dim3 grid(ceil_div(ncp, ppb), units);
  const size_t lds = (size_t(2) * G * c.d_k + 256) * sizeof(float);
  if (c.dtype == SE_F32)
    hipLaunchKernelGGL(quest_score_vector_kernel<float>, grid, dim3(256), lds, s, (const float*)q,
                       (const float*)kmin, (const float*)kmax, seq_len, score, c.n_kv_heads, G, c.d_k,
                       page_size, ncp);
  else
    hipLaunchKernelGGL(quest_score_vector_kernel<bf16_t>, grid, dim3(256), lds, s, (const bf16_t*)q,
                       (const bf16_t*)kmin, (const bf16_t*)kmax, seq_len, score, c.n_kv_heads, G, c.d_k,
                       page_size, ncp);
  if (hipGetLastError() != hipSuccess) return SE_ERR_HIP;
  hipLaunchKernelGGL(quest_topk_kernel<256>, dim3(units), dim3(256), 0, s, score, seq_len, view_idx,
                     view_len, c.n_kv_heads, page_size, ncp, top_pages);
  return launch_status();
}

}  // namespace se
