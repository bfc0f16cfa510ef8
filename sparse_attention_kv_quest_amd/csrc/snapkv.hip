// SnapKV prefill-end eviction (placeholder until the kernels land).
#include "se_internal.hpp"

namespace se {

size_t snapkv_ws_bytes(const se_cache& c, int prompt_len, int window) {
  return size_t(c.batch) * c.n_kv_heads * (prompt_len - window) * sizeof(float);
}

se_status launch_snapkv(const se_cache&, const void*, const void*, const void*, int, int, int, int, float,
                        const se_cache&, void*, void*, int32_t*, float*, int32_t*, void*, hipStream_t) {
  return SE_ERR_UNSUPPORTED;
}

}  // namespace se
