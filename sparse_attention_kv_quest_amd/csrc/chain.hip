// Chain Cache bookkeeping: logical prefixes and physical-row position maps.
//
// tokendh.com explainer, section "聊天记录也能'续命':Chain Cache": after a method
// has physically deleted part of a conversation's KV, the system still knows the
// logical prefix (the tokens that were said), keeps it apart from the rows it
// still stores, recognises a new turn that continues that prefix and computes
// only the new part.  Netics blog "SparseEngine 统一接入十五种稀疏注意力": the
// ChainCacheIndex ties a session to its retained per-layer KV, the method's
// metadata and the logical token prefix.  Here:
//  * matching is host logic over caller-owned session prefixes: the session
//    whose prefix the request continues, the longest such prefix, the lower
//    index on equal lengths;
//  * each unit keeps a map physical row -> logical position; a compaction that
//    keeps rows kept[0..n) composes it (map_out[i] = map_in[kept[i]]), and rows
//    appended after the retained ones take the next logical positions.
#include "se_internal.hpp"

namespace se {

void chain_match(const int32_t* tokens, int n_tokens, const int32_t* const* prefixes, const int32_t* lens,
                 int n_prefixes, int32_t* session, int32_t* matched) {
  int best = -1, blen = 0;
  for (int s = 0; s < n_prefixes; ++s) {
    const int n = lens[s];
    if (n > n_tokens || (best >= 0 && n <= blen)) continue;
    bool ok = true;
    for (int i = 0; i < n && ok; ++i) ok = prefixes[s][i] == tokens[i];
    if (ok) { best = s; blen = n; }
  }
  *session = best;
  *matched = blen;
}

// grid: units.  map_out[u][i] = map_in[u][kept[u][i]] (kept[u][i] itself without
// map_in) for i < kept_len[b], -1 for the rest of the unit's cap_out entries; a kept
// entry outside [0, cap_in) gives -1.
__global__ __launch_bounds__(256) void chain_remap_kernel(const int32_t* __restrict__ map_in, int cap_in,
                                                          const int32_t* __restrict__ kept, int kept_stride,
                                                          const int32_t* __restrict__ kept_len,
                                                          int32_t* __restrict__ map_out, int cap_out, int Hkv) {
  const int unit = blockIdx.x, b = unit / Hkv;
  const int n = min(max(kept_len[b], 0), min(kept_stride, cap_out));
  const int32_t* kr = kept + size_t(unit) * kept_stride;
  const int32_t* mr = map_in ? map_in + size_t(unit) * cap_in : nullptr;
  int32_t* orow = map_out + size_t(unit) * cap_out;
  for (int i = threadIdx.x; i < cap_out; i += blockDim.x) {
    int v = -1;
    if (i < n) {
      const int r = kr[i];
      if (r >= 0 && r < cap_in) v = mr ? mr[r] : r;
    }
    orow[i] = v;
  }
}

// grid: units.  Positions logical_len[b] + j of the rows j < n_new that follow the
// seq_len[b] retained physical rows (rows past cap are skipped).
__global__ __launch_bounds__(256) void chain_append_kernel(int32_t* __restrict__ pos_map, int cap,
                                                           const int32_t* __restrict__ seq_len,
                                                           const int32_t* __restrict__ logical_len, int n_new, int Hkv) {
  const int unit = blockIdx.x, b = unit / Hkv;
  const int p0 = seq_len[b];
  int32_t* row = pos_map + size_t(unit) * cap;
  for (int j = threadIdx.x; j < n_new; j += blockDim.x) {
    const int p = p0 + j;
    if (p >= 0 && p < cap) row[p] = logical_len[b] + j;
  }
}

se_status launch_chain_remap(const se_cache& c, const int32_t* map_in, int cap_in, const int32_t* kept,
                             int kept_stride, const int32_t* kept_len, int32_t* map_out, hipStream_t s) {
  hipLaunchKernelGGL(chain_remap_kernel, dim3(c.batch * c.n_kv_heads), dim3(256), 0, s, map_in, cap_in, kept,
                     kept_stride, kept_len, map_out, c.capacity, c.n_kv_heads);
  return launch_status();
}

se_status launch_chain_append(const se_cache& c, int32_t* pos_map, const int32_t* seq_len, const int32_t* logical_len,
                              int n_new, hipStream_t s) {
  hipLaunchKernelGGL(chain_append_kernel, dim3(c.batch * c.n_kv_heads), dim3(256), 0, s, pos_map, c.capacity, seq_len,
                     logical_len, n_new, c.n_kv_heads);
  return launch_status();
}

}  // namespace se
