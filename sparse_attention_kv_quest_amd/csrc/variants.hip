// StreamingLLM views and PyramidKV layer budgets.
//
// Netics blog "SparseEngine 统一接入十五种稀疏注意力", section
// "哪些情况下加速幅度会缩小": the paper compares StreamingLLM and PyramidKV with
// SnapKV on AIME 2024; the pages name the two methods and nothing more.  Their
// plainest forms over this library's cache contract:
//  * StreamingLLM attends over the first `sink` and the last `recent` positions
//    of a unit's history: a token view handed to the decode attention, no data
//    moved;
//  * PyramidKV gives deeper layers smaller budgets along an arithmetic sequence
//    whose mean is the average budget, each layer then selecting as SnapKV does
//    (the SnapKV call with that layer's budget).  The schedule is host logic.
#include <algorithm>
#include <vector>

#include "se_internal.hpp"

namespace se {

// grid: units; every entry e < view_cap of the unit's row: positions [0, sink)
// then [len - recent, len), ascending, -1 past the kept count.
__global__ __launch_bounds__(256) void streaming_view_kernel(const int32_t* __restrict__ seq_len,
                                                             int32_t* __restrict__ view_idx,
                                                             int32_t* __restrict__ view_len, int Hkv, int cap,
                                                             int sink, int recent, int view_cap, int pending) {
  const int unit = blockIdx.x, b = unit / Hkv;
  const int len = int(min(int64_t(max(seq_len[b], 0)) + pending, int64_t(cap)));   // after `pending` appends
  const int n_head = min(sink, len);
  const int tail0 = max(n_head, len - recent);    // first recent position not already in the sink
  const int n = n_head + (len - tail0);
  int32_t* row = view_idx + size_t(unit) * view_cap;
  for (int e = threadIdx.x; e < view_cap; e += blockDim.x)
    row[e] = e < n_head ? e : (e < n ? tail0 + (e - n_head) : -1);
  if (threadIdx.x == 0) view_len[unit] = n;
}

se_status launch_streaming_view(const se_cache& c, const int32_t* seq_len, int sink, int recent,
                                int32_t* view_idx, int32_t* view_len, int view_cap, int pending, hipStream_t s) {
  hipLaunchKernelGGL(streaming_view_kernel, dim3(c.batch * c.n_kv_heads), dim3(256), 0, s, seq_len, view_idx,
                     view_len, c.n_kv_heads, c.capacity, sink, recent, view_cap, pending);
  return launch_status();
}

// Budget of layer l (0 = first): b_min + (b_max - b_min) (n - 1 - l) / (n - 1) with
// b_max = 2 avg - b_min, in whole tokens summing to n * avg: floors first, then one
// more token to each of the layers with the largest remainders (lower layer first
// on equal remainders).  Integer arithmetic throughout, so the schedule is exact.
void pyramid_budgets(int n, int avg, int bmin, int32_t* out) {
  if (n == 1) {
    out[0] = avg;
    return;
  }
  const int64_t den = n - 1, span = 2 * int64_t(avg) - 2 * int64_t(bmin);   // b_max - b_min
  std::vector<int64_t> rem(n);
  int64_t total = 0;
  for (int l = 0; l < n; ++l) {
    const int64_t num = span * (n - 1 - l);
    out[l] = int32_t(bmin + num / den);
    rem[l] = num % den;
    total += out[l];
  }
  std::vector<int> order(n);
  for (int l = 0; l < n; ++l) order[l] = l;
  std::stable_sort(order.begin(), order.end(), [&](int x, int y) { return rem[x] > rem[y]; });
  const int64_t left = int64_t(n) * avg - total;
  for (int64_t i = 0; i < left; ++i) out[order[i]] += 1;
}

}  // namespace se
