// C ABI of libse: host-side validation, then dispatch to the launchers.
// Nothing is enqueued unless every argument checks out.
#include "se_internal.hpp"
#include <stdio.h>
#include <stdlib.h>

#include <mutex>
#include <vector>

using namespace se;

namespace {

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Launch failures are read back with hipGetLastError after the launches; an
// error left by an earlier, unrelated HIP call is cleared first so that it is
// not reported as this call's.
void clear_stale_error() { (void)hipGetLastError(); }

bool trace_on() {
  static int on = -1;
  if (on < 0) {
    const char* e = getenv("SE_TRACE");
    on = (e && e[0] && e[0] != '0') ? 1 : 0;
  }
  return on == 1;
}

// Debug mode (SE_CHECK_VIEWS=1 in the environment, read once): the attention calls
// synchronise the stream, copy the view and its lengths to the host and check every
// entry in use (view_len within [0, view_cap], each entry >= 0 with its first slot
// inside the cache's capacity; entries past seq_len are allowed, their slots are
// skipped) before launching; a bad view returns SE_ERR_SHAPE and launches nothing.
// Not for graph capture.
bool check_views_on() {
  static int on = -1;
  if (on < 0) {
    const char* e = getenv("SE_CHECK_VIEWS");
    on = (e && e[0] && e[0] != '0') ? 1 : 0;
  }
  return on == 1;
}

se_status check_view_host(const se_cache* c, const int32_t* view_idx, const int32_t* view_len, int32_t view_cap,
                          int32_t granularity, hipStream_t stream) {
  const int units = c->batch * c->n_kv_heads;
  std::vector<int32_t> v(size_t(units) * view_cap), vl(units);
  if (hipStreamSynchronize(stream) != hipSuccess ||
      hipMemcpy(v.data(), view_idx, v.size() * sizeof(int32_t), hipMemcpyDeviceToHost) != hipSuccess ||
      hipMemcpy(vl.data(), view_len, vl.size() * sizeof(int32_t), hipMemcpyDeviceToHost) != hipSuccess)
    return SE_ERR_HIP;
  for (int u = 0; u < units; ++u) {
    const int n = vl[u];
    if (n < 0 || n > view_cap) return SE_ERR_SHAPE;
    for (int e = 0; e < n; ++e) {
      const int32_t x = v[size_t(u) * view_cap + e];
      if (x < 0 || int64_t(x) * granularity >= c->capacity) return SE_ERR_SHAPE;
    }
  }
  return SE_OK;
}

#define SE_TRACE_CALL(...)                                  \
  do {                                                      \
    if (trace_on()) { fprintf(stderr, "[se] " __VA_ARGS__); fputc('\n', stderr); } \
  } while (0)

se_status check_cache(const se_cache* c) {
  if (c == nullptr) return SE_ERR_NULL;
  if (c->dtype != SE_F32 && c->dtype != SE_BF16) return SE_ERR_DTYPE;
  if (c->batch <= 0 || c->n_q_heads <= 0 || c->n_kv_heads <= 0 || c->capacity <= 0) return SE_ERR_SHAPE;
  if (c->n_q_heads % c->n_kv_heads != 0) return SE_ERR_SHAPE;
  if (c->n_q_heads / c->n_kv_heads > 64) return SE_ERR_SHAPE;
  if (c->d_k != 64 && c->d_k != 128 && c->d_k != 576) return SE_ERR_SHAPE;
  if (c->latent) {
    if (c->n_kv_heads != 1 || c->d_v <= 0 || c->d_v > c->d_k || c->d_v % 8 != 0) return SE_ERR_SHAPE;
  } else if (c->d_v != c->d_k) {
    return SE_ERR_SHAPE;
  }
  return SE_OK;
}

// Argument checks of the attention calls (cache already checked), up to the
// workspace size, which the caller compares: *need receives it.
se_status attn_validate(const se_cache* c, const void* q, const void* k, const void* v, const int32_t* seq_len,
                        const int32_t* view_idx, const int32_t* view_len, int32_t view_cap, int32_t granularity,
                        float scale, float* out, float* logits, int32_t logit_cap, int32_t num_splits,
                        size_t* need) {
  if (!q || !k || !seq_len || !out || (!c->latent && !v)) return SE_ERR_NULL;
  if (!aligned16(q) || !aligned16(k) || (!c->latent && !aligned16(v)) || !aligned16(out)) return SE_ERR_ALIGN;
  if (view_idx) {
    if (!view_len) return SE_ERR_NULL;
    if (view_cap <= 0 || granularity <= 0) return SE_ERR_SHAPE;
    if (int64_t(view_cap) * granularity > (int64_t(1) << 30)) return SE_ERR_SHAPE;
  }
  if (logits && logit_cap <= 0) return SE_ERR_SHAPE;
  // a group's logit rows are addressed with 32-bit offsets
  if (logits && int64_t(c->n_q_heads / c->n_kv_heads) * logit_cap > INT32_MAX) return SE_ERR_SHAPE;
  if (num_splits < 0 || num_splits > 256) return SE_ERR_SHAPE;
  if (!(scale > 0.f) || !(scale < 1e30f)) return SE_ERR_SHAPE;
  const int slots = view_idx ? view_cap * granularity : c->capacity;
  *need = attn_ws_bytes(*c, slots, num_splits);
  return SE_OK;
}

// Shared validation and launch of the attention calls (cache already checked);
// k_scale / v_scale non-null for FP8 rows.
se_status attn_impl(const se_cache* c, const void* q, const void* k, const void* v, const int32_t* seq_len,
                    const int32_t* view_idx, const int32_t* view_len, int32_t view_cap, int32_t granularity,
                    float scale, float* out, float* lse, float* logits, int32_t logit_cap, int32_t num_splits,
                    void* ws, size_t ws_bytes, hipStream_t stream, const uint8_t* k_scale, const uint8_t* v_scale) {
  size_t need = 0;
  se_status st = attn_validate(c, q, k, v, seq_len, view_idx, view_len, view_cap, granularity, scale, out, logits,
                               logit_cap, num_splits, &need);
  if (st != SE_OK) return st;
  if (!ws || ws_bytes < need) return SE_ERR_WORKSPACE;
  if (view_idx && check_views_on()) {
    st = check_view_host(c, view_idx, view_len, view_cap, granularity, stream);
    if (st != SE_OK) return st;
  }
  SE_TRACE_CALL("sparse_decode_attn%s B=%d Hq=%d Hkv=%d d_k=%d d_v=%d view=%s cap=%d g=%d splits=%d logits=%d",
                k_scale ? "_fp8" : "", c->batch, c->n_q_heads, c->n_kv_heads, c->d_k, c->d_v, view_idx ? "idx" : "identity",
                view_cap, granularity, num_splits, logits ? logit_cap : 0);
  clear_stale_error();
  return launch_attn(*c, q, k, v, seq_len, view_idx, view_len, view_cap, granularity, scale, out, lse, logits,
                     logit_cap, num_splits, ws, stream, k_scale, v_scale);
}

// Device memory of se_sparse_decode_attn_noalloc: one array per GPU the library
// runs on, held until the process ends.  In host code `scratch` names a host-side
// stand-in, never the device array: kernels and fills get the address that
// hipGetSymbolAddress returns for the current device.
static __device__ __align__(256) unsigned char scratch[SE_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// The scratch array's device address on the current device, looked up once per device.
se_status scratch_of_current_device(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return SE_ERR_HIP;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) return SE_ERR_HIP;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return SE_OK;
}

}  // namespace

extern "C" {

int32_t se_abi_version(void) { return SE_ABI_VERSION; }

const char* se_status_string(int32_t st) {
  switch (st) {
    case SE_OK: return "ok";
    case SE_ERR_NULL: return "null pointer";
    case SE_ERR_SHAPE: return "bad shape";
    case SE_ERR_DTYPE: return "unsupported dtype";
    case SE_ERR_ALIGN: return "pointer not 16-byte aligned";
    case SE_ERR_BUDGET: return "budget / window / k out of range";
    case SE_ERR_WORKSPACE: return "workspace too small";
    case SE_ERR_UNSUPPORTED: return "unsupported combination";
    case SE_ERR_HIP: return "HIP launch failed";
    default: return "unknown status";
  }
}

size_t se_workspace_bytes(int32_t op, const se_cache* c, int32_t a0, int32_t a1) {
  if (check_cache(c) != SE_OK) return 0;
  switch (op) {
    case SE_OP_QUEST: return a0 > 0 ? quest_ws_bytes(*c, a0, a1) : 0;
    case SE_OP_ATTN: return attn_ws_bytes(*c, a0 > 0 ? a0 : c->capacity, a1);
    case SE_OP_SNAPKV: return (a0 > a1 && a1 > 0) ? snapkv_ws_bytes(*c, a0, a1) : 0;
    case SE_OP_OMNIKV: return a0 > 0 ? omnikv_ws_bytes(*c, a0, a1) : 0;
    case SE_OP_QUEST_APPEND: return a0 > 0 ? quest_append_ws_bytes(*c, a0) : 0;
    case SE_OP_H2O_PREFILL: return (a0 > a1 && a1 > 0) ? h2o_prefill_ws_bytes(*c, a0, a1) : 0;
    case SE_OP_APPEND_ATTN: return attn_append_ws_bytes(*c, a0 > 0 ? a0 : c->capacity, a1);
    case SE_OP_QUEST_STEP: return (a0 > 0 && a1 > 0) ? quest_step_ws_bytes(*c, a0, a1) : 0;
    case SE_OP_H2O_STEP: return h2o_step_ws_bytes(*c);
    default: return 0;
  }
}

se_status se_workspace_init(void* ws, size_t bytes, hipStream_t stream) {
  SE_TRACE_CALL("workspace_init bytes=%zu", bytes);
  if (bytes == 0) return SE_OK;
  if (!ws) return SE_ERR_NULL;
  if (!aligned16(ws)) return SE_ERR_ALIGN;
  clear_stale_error();
  return launch_zero_fill(ws, bytes, stream);
}

se_status se_kv_append(const se_cache* c, void* k, void* v, const void* k_new, const void* v_new,
                       const int32_t* slot, int32_t* seq_len, hipStream_t stream) {
  se_status st = check_cache(c);
  if (st != SE_OK) return st;
  if (!k || !k_new || !seq_len || (!c->latent && (!v || !v_new))) return SE_ERR_NULL;
  if (!aligned16(k) || !aligned16(k_new) || (!c->latent && (!aligned16(v) || !aligned16(v_new))))
    return SE_ERR_ALIGN;
  SE_TRACE_CALL("kv_append B=%d Hkv=%d d_k=%d cap=%d slot=%p", c->batch, c->n_kv_heads, c->d_k, c->capacity,
                (const void*)slot);
  clear_stale_error();
  return launch_kv_append(*c, k, v, k_new, v_new, slot, seq_len, stream);
}

se_status se_kv_append_meta(const se_cache* c, void* k, void* v, const void* k_new, const void* v_new,
                            const int32_t* slot, int32_t* seq_len, void* kmin, void* kmax, int32_t page_size,
                            hipStream_t stream) {
  se_status st = check_cache(c);
  if (st != SE_OK) return st;
  if (!k || !k_new || !seq_len || !kmin || !kmax || (!c->latent && (!v || !v_new))) return SE_ERR_NULL;
  if (!aligned16(k) || !aligned16(k_new) || !aligned16(kmin) || !aligned16(kmax) ||
      (!c->latent && (!aligned16(v) || !aligned16(v_new))))
    return SE_ERR_ALIGN;
  if (page_size <= 0 || page_size > c->capacity) return SE_ERR_SHAPE;
  SE_TRACE_CALL("kv_append_meta B=%d Hkv=%d d_k=%d cap=%d P=%d slot=%p", c->batch, c->n_kv_heads, c->d_k,
                c->capacity, page_size, (const void*)slot);
  clear_stale_error();
  return launch_kv_append_meta(*c, k, v, k_new, v_new, slot, seq_len, kmin, kmax, page_size, stream);
}

se_status se_page_meta_update(const se_cache* c, const void* k, void* kmin, void* kmax,
                              const int32_t* seq_len, int32_t page_size, int32_t first_page,
                              hipStream_t stream) {
  se_status st = check_cache(c);
  if (st != SE_OK) return st;
  if (!k || !kmin || !kmax || !seq_len) return SE_ERR_NULL;
  if (!aligned16(k) || !aligned16(kmin) || !aligned16(kmax)) return SE_ERR_ALIGN;
  if (page_size <= 0 || page_size > c->capacity || first_page < -1) return SE_ERR_SHAPE;
  SE_TRACE_CALL("page_meta B=%d Hkv=%d d_k=%d P=%d first=%d", c->batch, c->n_kv_heads, c->d_k, page_size,
                first_page);
  clear_stale_error();
  return launch_page_meta(*c, k, kmin, kmax, seq_len, page_size, first_page, stream);
}

se_status se_quest_select(const se_cache* c, const void* q, const void* kmin, const void* kmax,
                          const int32_t* seq_len, int32_t page_size, int32_t top_pages,
                          int32_t* view_idx, int32_t* view_len, float* page_score,
                          void* ws, size_t ws_bytes, hipStream_t stream) {
  se_status st = check_cache(c);
  if (st != SE_OK) return st;
  if (!q || !kmin || !kmax || !seq_len || !view_idx || !view_len) return SE_ERR_NULL;
  if (!aligned16(q) || !aligned16(kmin) || !aligned16(kmax)) return SE_ERR_ALIGN;
  if (page_size <= 0 || page_size > c->capacity) return SE_ERR_SHAPE;
  if (top_pages < 1) return SE_ERR_BUDGET;
  if (!page_score) {
    const size_t need = quest_ws_bytes(*c, page_size, top_pages);
    if (!ws || ws_bytes < need) return SE_ERR_WORKSPACE;
  }
  SE_TRACE_CALL("quest_select B=%d Hq=%d Hkv=%d d_k=%d P=%d k=%d", c->batch, c->n_q_heads, c->n_kv_heads,
                c->d_k, page_size, top_pages);
  clear_stale_error();
  return launch_quest(*c, q, kmin, kmax, seq_len, page_size, top_pages, view_idx, view_len, page_score, ws,
                      stream);
}

se_status se_quest_append_select(const se_cache* c, const void* q, void* k, void* v, const void* k_new,
                                 const void* v_new, int32_t* seq_len, void* kmin, void* kmax, int32_t page_size,
                                 int32_t top_pages, int32_t* view_idx, int32_t* view_len, float* page_score,
                                 void* ws, size_t ws_bytes, hipStream_t stream) {
  se_status st = check_cache(c);
  if (st != SE_OK) return st;
  if (!q || !k || !k_new || !seq_len || !kmin || !kmax || !view_idx || !view_len || !ws ||
      (!c->latent && (!v || !v_new)))
    return SE_ERR_NULL;
  if (!aligned16(q) || !aligned16(k) || !aligned16(k_new) || !aligned16(kmin) || !aligned16(kmax) || !aligned16(ws) ||
      (!c->latent && (!aligned16(v) || !aligned16(v_new))))
    return SE_ERR_ALIGN;
  if (page_size <= 0 || page_size > c->capacity) return SE_ERR_SHAPE;
  if (top_pages < 1) return SE_ERR_BUDGET;
  if (ws_bytes < quest_append_ws_bytes(*c, page_size)) return SE_ERR_WORKSPACE;
  SE_TRACE_CALL("quest_append_select B=%d Hq=%d Hkv=%d d_k=%d P=%d k=%d", c->batch, c->n_q_heads, c->n_kv_heads,
                c->d_k, page_size, top_pages);
  clear_stale_error();
  return launch_quest_append(*c, q, k, v, k_new, v_new, seq_len, kmin, kmax, page_size, top_pages, view_idx,
                             view_len, page_score, ws, stream);
}

se_status se_quest_decode_step(const se_cache* c, const void* q, void* k, void* v, const void* k_new,
                               const void* v_new, int32_t* seq_len, void* kmin, void* kmax, int32_t page_size,
                               int32_t top_pages, float scale, float* out, float* lse, int32_t* view_idx,
                               int32_t* view_len, float* page_score, void* ws, size_t ws_bytes, hipStream_t stream) {
  se_status st = check_cache(c);
  if (st != SE_OK) return st;
  if (!q || !k || !k_new || !seq_len || !kmin || !kmax || !out || !ws || (!c->latent && (!v || !v_new)))
    return SE_ERR_NULL;
  if ((view_idx == nullptr) != (view_len == nullptr)) return SE_ERR_NULL;
  if (!aligned16(q) || !aligned16(k) || !aligned16(k_new) || !aligned16(kmin) || !aligned16(kmax) || !aligned16(ws) ||
      !aligned16(out) || (!c->latent && (!aligned16(v) || !aligned16(v_new))))
    return SE_ERR_ALIGN;
  if (page_size <= 0 || page_size > c->capacity) return SE_ERR_SHAPE;
  if (top_pages < 1) return SE_ERR_BUDGET;
  if (int64_t(top_pages) * page_size > (int64_t(1) << 30)) return SE_ERR_SHAPE;
  if (!(scale > 0.f) || !(scale < 1e30f)) return SE_ERR_SHAPE;
  if (ws_bytes < quest_step_ws_bytes(*c, page_size, top_pages)) return SE_ERR_WORKSPACE;
  SE_TRACE_CALL("quest_decode_step B=%d Hq=%d Hkv=%d d_k=%d P=%d k=%d", c->batch, c->n_q_heads, c->n_kv_heads,
                c->d_k, page_size, top_pages);
  clear_stale_error();
  return launch_quest_step(*c, q, k, v, k_new, v_new, seq_len, kmin, kmax, page_size, top_pages, scale, out, lse,
                           view_idx, view_len, page_score, ws, stream);
}

// FP8 caches: bf16 q / metadata / source rows, GQA with d_k 64 or 128.
se_status check_fp8_cache(const se_cache* c) {
  se_status st = check_cache(c);
  if (st != SE_OK) return st;
  if (c->dtype != SE_BF16) return SE_ERR_DTYPE;
  if (c->latent || (c->d_k != 64 && c->d_k != 128)) return SE_ERR_UNSUPPORTED;
  return SE_OK;
}

se_status se_quest_decode_step_fp8(const se_cache* c, const void* q, void* k_q, void* v_q, uint8_t* k_scale,
                                   uint8_t* v_scale, const void* k_new, const void* v_new, int32_t* seq_len,
                                   void* kmin, void* kmax, int32_t page_size, int32_t top_pages, float scale,
                                   float* out, float* lse, int32_t* view_idx, int32_t* view_len, float* page_score,
                                   void* ws, size_t ws_bytes, hipStream_t stream) {
  se_status st = check_fp8_cache(c);
  if (st != SE_OK) return st;
  if (c->n_q_heads / c->n_kv_heads > 16) return SE_ERR_UNSUPPORTED;
  if (!q || !k_q || !v_q || !k_scale || !v_scale || !k_new || !v_new || !seq_len || !kmin || !kmax || !out || !ws)
    return SE_ERR_NULL;
  if ((view_idx == nullptr) != (view_len == nullptr)) return SE_ERR_NULL;
  if (!aligned16(q) || !aligned16(k_q) || !aligned16(v_q) || !aligned16(k_new) || !aligned16(v_new) ||
      !aligned16(kmin) || !aligned16(kmax) || !aligned16(ws) || !aligned16(out))
    return SE_ERR_ALIGN;
  if (page_size <= 0 || page_size > c->capacity) return SE_ERR_SHAPE;
  if (top_pages < 1) return SE_ERR_BUDGET;
  if (int64_t(top_pages) * page_size > (int64_t(1) << 30)) return SE_ERR_SHAPE;
  if (!(scale > 0.f) || !(scale < 1e30f)) return SE_ERR_SHAPE;
  if (ws_bytes < quest_step_ws_bytes(*c, page_size, top_pages)) return SE_ERR_WORKSPACE;
  SE_TRACE_CALL("quest_decode_step_fp8 B=%d Hq=%d Hkv=%d d_k=%d P=%d k=%d", c->batch, c->n_q_heads, c->n_kv_heads,
                c->d_k, page_size, top_pages);
  clear_stale_error();
  return launch_quest_step_fp8(*c, q, k_q, v_q, k_scale, v_scale, k_new, v_new, seq_len, kmin, kmax, page_size,
                               top_pages, scale, out, lse, view_idx, view_len, page_score, ws, stream);
}

se_status se_kv_quantize_fp8(const se_cache* c, const void* k, const void* v, const int32_t* seq_len, void* k_q,
                             void* v_q, uint8_t* k_scale, uint8_t* v_scale, void* kmin, void* kmax, int32_t page_size,
                             hipStream_t stream) {
  se_status st = check_fp8_cache(c);
  if (st != SE_OK) return st;
  if (!k || !v || !seq_len || !k_q || !v_q || !k_scale || !v_scale || (!kmin != !kmax)) return SE_ERR_NULL;
  if (!aligned16(k) || !aligned16(v) || !aligned16(k_q) || !aligned16(v_q) ||
      (kmin && (!aligned16(kmin) || !aligned16(kmax))))
    return SE_ERR_ALIGN;
  if (kmin && (page_size <= 0 || page_size > c->capacity)) return SE_ERR_SHAPE;
  SE_TRACE_CALL("kv_quantize_fp8 B=%d Hkv=%d d_k=%d cap=%d", c->batch, c->n_kv_heads, c->d_k, c->capacity);
  clear_stale_error();
  return launch_fp8_quantize(*c, k, v, seq_len, k_q, v_q, k_scale, v_scale, kmin, kmax, page_size, stream);
}

se_status se_kv_append_fp8(const se_cache* c, void* k_q, void* v_q, uint8_t* k_scale, uint8_t* v_scale,
                           const void* k_new, const void* v_new, int32_t* seq_len, void* kmin, void* kmax,
                           int32_t page_size, hipStream_t stream) {
  se_status st = check_fp8_cache(c);
  if (st != SE_OK) return st;
  if (!k_q || !v_q || !k_scale || !v_scale || !k_new || !v_new || !seq_len || (!kmin != !kmax)) return SE_ERR_NULL;
  if (!aligned16(k_q) || !aligned16(v_q) || !aligned16(k_new) || !aligned16(v_new) ||
      (kmin && (!aligned16(kmin) || !aligned16(kmax))))
    return SE_ERR_ALIGN;
  if (page_size <= 0 || page_size > c->capacity) return SE_ERR_SHAPE;
  SE_TRACE_CALL("kv_append_fp8 B=%d Hkv=%d d_k=%d cap=%d P=%d", c->batch, c->n_kv_heads, c->d_k, c->capacity,
                page_size);
  clear_stale_error();
  return launch_fp8_append(*c, k_q, v_q, k_scale, v_scale, k_new, v_new, seq_len, kmin, kmax, page_size, stream);
}

se_status se_sparse_decode_attn_fp8(const se_cache* c, const void* q, const void* k_q, const void* v_q,
                                    const uint8_t* k_scale, const uint8_t* v_scale, const int32_t* seq_len,
                                    const int32_t* view_idx, const int32_t* view_len, int32_t view_cap,
                                    int32_t granularity, float scale, float* out, float* lse, float* logits,
                                    int32_t logit_cap, int32_t num_splits, void* ws, size_t ws_bytes,
                                    hipStream_t stream) {
  se_status st = check_fp8_cache(c);
  if (st != SE_OK) return st;
  if (c->n_q_heads / c->n_kv_heads > 16) return SE_ERR_UNSUPPORTED;
  if (!k_scale || !v_scale || !v_q) return SE_ERR_NULL;
  return attn_impl(c, q, k_q, v_q, seq_len, view_idx, view_len, view_cap, granularity, scale, out, lse, logits,
                   logit_cap, num_splits, ws, ws_bytes, stream, k_scale, v_scale);
}

se_status se_streaming_view(const se_cache* c, const int32_t* seq_len, int32_t sink, int32_t recent,
                            int32_t* view_idx, int32_t* view_len, int32_t view_cap, int32_t pending,
                            hipStream_t stream) {
  se_status st = check_cache(c);
  if (st != SE_OK) return st;
  if (!seq_len || !view_idx || !view_len) return SE_ERR_NULL;
  if (sink < 0 || recent < 0 || int64_t(sink) + recent < 1 || view_cap < int64_t(sink) + recent)
    return SE_ERR_BUDGET;
  if (pending < 0 || pending > c->capacity) return SE_ERR_SHAPE;
  SE_TRACE_CALL("streaming_view B=%d Hkv=%d sink=%d recent=%d cap=%d", c->batch, c->n_kv_heads, sink, recent,
                view_cap);
  clear_stale_error();
  return launch_streaming_view(*c, seq_len, sink, recent, view_idx, view_len, view_cap, pending, stream);
}

se_status se_chain_match(const int32_t* tokens, int32_t n_tokens, const int32_t* const* prefixes,
                         const int32_t* prefix_lens, int32_t n_prefixes, int32_t* session, int32_t* matched_len) {
  if (!session || !matched_len) return SE_ERR_NULL;
  if (n_tokens < 0 || n_prefixes < 0) return SE_ERR_SHAPE;
  if ((n_tokens > 0 && !tokens) || (n_prefixes > 0 && (!prefixes || !prefix_lens))) return SE_ERR_NULL;
  for (int s = 0; s < n_prefixes; ++s) {
    if (prefix_lens[s] < 0) return SE_ERR_SHAPE;
    if (prefix_lens[s] > 0 && !prefixes[s]) return SE_ERR_NULL;
  }
  chain_match(tokens, n_tokens, prefixes, prefix_lens, n_prefixes, session, matched_len);
  return SE_OK;
}

se_status se_chain_remap(const se_cache* c_out, const int32_t* map_in, int32_t cap_in, const int32_t* kept,
                         int32_t kept_stride, const int32_t* kept_len, int32_t* map_out, hipStream_t stream) {
  se_status st = check_cache(c_out);
  if (st != SE_OK) return st;
  if (!kept || !kept_len || !map_out) return SE_ERR_NULL;
  if (kept_stride < 1 || (map_in && cap_in < 1)) return SE_ERR_SHAPE;
  SE_TRACE_CALL("chain_remap B=%d Hkv=%d cap_out=%d stride=%d", c_out->batch, c_out->n_kv_heads, c_out->capacity,
                kept_stride);
  clear_stale_error();
  return launch_chain_remap(*c_out, map_in, map_in ? cap_in : 0x7fffffff, kept, kept_stride, kept_len, map_out,
                            stream);
}

se_status se_chain_append_positions(const se_cache* c, int32_t* pos_map, const int32_t* seq_len,
                                    const int32_t* logical_len, int32_t n_new, hipStream_t stream) {
  se_status st = check_cache(c);
  if (st != SE_OK) return st;
  if (!pos_map || !seq_len || !logical_len) return SE_ERR_NULL;
  if (n_new < 0) return SE_ERR_SHAPE;
  if (n_new == 0) return SE_OK;
  clear_stale_error();
  return launch_chain_append(*c, pos_map, seq_len, logical_len, n_new, stream);
}

se_status se_pyramid_budgets(int32_t n_layers, int32_t avg_budget, int32_t min_budget, int32_t* budgets) {
  if (!budgets) return SE_ERR_NULL;
  if (n_layers < 1) return SE_ERR_SHAPE;
  if (min_budget < 0 || min_budget > avg_budget) return SE_ERR_BUDGET;
  pyramid_budgets(n_layers, avg_budget, min_budget, budgets);
  return SE_OK;
}

se_status se_sparse_decode_attn(const se_cache* c, const void* q, const void* k, const void* v,
                                const int32_t* seq_len, const int32_t* view_idx,
                                const int32_t* view_len, int32_t view_cap, int32_t granularity,
                                float scale, float* out, float* lse, float* logits,
                                int32_t logit_cap, int32_t num_splits,
                                void* ws, size_t ws_bytes, hipStream_t stream) {
  se_status st = check_cache(c);
  if (st != SE_OK) return st;
  return attn_impl(c, q, k, v, seq_len, view_idx, view_len, view_cap, granularity, scale, out, lse, logits, logit_cap,
                   num_splits, ws, ws_bytes, stream, nullptr, nullptr);
}

se_status se_sparse_decode_attn_noalloc(const se_cache* c, const void* q, const void* k, const void* v,
                                        const int32_t* seq_len, const int32_t* view_idx,
                                        const int32_t* view_len, int32_t view_cap, int32_t granularity,
                                        float scale, float* out, float* lse, float* logits,
                                        int32_t logit_cap, int32_t num_splits, hipStream_t stream) {
  se_status st = check_cache(c);
  if (st != SE_OK) return st;
  size_t need = 0;
  st = attn_validate(c, q, k, v, seq_len, view_idx, view_len, view_cap, granularity, scale, out, logits, logit_cap,
                     num_splits, &need);
  if (st != SE_OK) return st;
  if (need > SE_NOALLOC_SCRATCH_BYTES) return SE_ERR_WORKSPACE;
  void* ws = nullptr;
  clear_stale_error();
  st = scratch_of_current_device(&ws);
  if (st != SE_OK) return st;
  SE_TRACE_CALL("sparse_decode_attn_noalloc B=%d Hq=%d Hkv=%d d_k=%d view=%s cap=%d g=%d splits=%d scratch=%zu",
                c->batch, c->n_q_heads, c->n_kv_heads, c->d_k, view_idx ? "idx" : "identity", view_cap, granularity,
                num_splits, need);
  // the ticket counters start at zero: cleared by a fill kernel (capturable) on the
  // caller's stream, ahead of the attention, whatever an earlier call left there
  st = launch_zero_fill(ws, attn_counter_bytes(*c), stream);
  if (st != SE_OK) return st;
  return launch_attn(*c, q, k, v, seq_len, view_idx, view_len, view_cap, granularity, scale, out, lse, logits,
                     logit_cap, num_splits, ws, stream, nullptr, nullptr);
}

se_status se_kv_append_decode_attn(const se_cache* c, const void* q, void* k, void* v, const void* k_new,
                                   const void* v_new, const int32_t* slot, int32_t* seq_len,
                                   const int32_t* view_idx, const int32_t* view_len, int32_t view_cap,
                                   int32_t granularity, float scale, float* out, float* lse, float* logits,
                                   int32_t logit_cap, int32_t num_splits, void* ws, size_t ws_bytes,
                                   hipStream_t stream) {
  se_status st = check_cache(c);
  if (st != SE_OK) return st;
  if (!q || !k || !k_new || !seq_len || !out || (!c->latent && (!v || !v_new))) return SE_ERR_NULL;
  if (!aligned16(q) || !aligned16(k) || !aligned16(k_new) || !aligned16(out) ||
      (!c->latent && (!aligned16(v) || !aligned16(v_new))))
    return SE_ERR_ALIGN;
  if (view_idx) {
    if (!view_len) return SE_ERR_NULL;
    if (view_cap <= 0 || granularity <= 0) return SE_ERR_SHAPE;
    if (int64_t(view_cap) * granularity > (int64_t(1) << 30)) return SE_ERR_SHAPE;
  }
  if (logits && logit_cap <= 0) return SE_ERR_SHAPE;
  // a group's logit rows are addressed with 32-bit offsets
  if (logits && int64_t(c->n_q_heads / c->n_kv_heads) * logit_cap > INT32_MAX) return SE_ERR_SHAPE;
  if (num_splits < 0 || num_splits > 256) return SE_ERR_SHAPE;
  if (!(scale > 0.f) || !(scale < 1e30f)) return SE_ERR_SHAPE;
  const int slots = view_idx ? view_cap * granularity : c->capacity;
  if (!ws || ws_bytes < attn_append_ws_bytes(*c, slots, num_splits)) return SE_ERR_WORKSPACE;
  SE_TRACE_CALL("kv_append_decode_attn B=%d Hq=%d Hkv=%d d_k=%d view=%s cap=%d g=%d splits=%d slot=%p logits=%d",
                c->batch, c->n_q_heads, c->n_kv_heads, c->d_k, view_idx ? "idx" : "identity", view_cap, granularity,
                num_splits, (const void*)slot, logits ? logit_cap : 0);
  clear_stale_error();
  return launch_append_attn(*c, q, k, v, k_new, v_new, slot, seq_len, view_idx, view_len, view_cap, granularity,
                            scale, out, lse, logits, logit_cap, num_splits, ws, stream);
}

se_status se_snapkv_score_compact(const se_cache* c, const void* q_obs, const void* k, const void* v,
                                  int32_t prompt_len, int32_t window, int32_t pool_kernel,
                                  int32_t budget, float scale, const se_cache* out, void* k_out,
                                  void* v_out, int32_t* kept_pos, float* votes,
                                  int32_t* out_seq_len, void* ws, size_t ws_bytes,
                                  hipStream_t stream) {
  se_status st = check_cache(c);
  if (st != SE_OK) return st;
  st = check_cache(out);
  if (st != SE_OK) return st;
  if (!q_obs || !k || !k_out || !kept_pos || (!c->latent && (!v || !v_out))) return SE_ERR_NULL;
  if (!aligned16(q_obs) || !aligned16(k) || !aligned16(k_out) ||
      (!c->latent && (!aligned16(v) || !aligned16(v_out))))
    return SE_ERR_ALIGN;
  if (c->latent) return SE_ERR_UNSUPPORTED;
  if (out->batch != c->batch || out->n_q_heads != c->n_q_heads || out->n_kv_heads != c->n_kv_heads ||
      out->d_k != c->d_k || out->d_v != c->d_v || out->dtype != c->dtype || out->latent != c->latent)
    return SE_ERR_SHAPE;
  if (prompt_len <= 0 || prompt_len > c->capacity) return SE_ERR_SHAPE;
  if (window < 1 || window >= prompt_len) return SE_ERR_BUDGET;
  if (pool_kernel < 1 || pool_kernel % 2 == 0 || pool_kernel > 129) return SE_ERR_BUDGET;
  if (budget < window) return SE_ERR_BUDGET;
  if (out->capacity < std::min(budget, prompt_len)) return SE_ERR_BUDGET;
  if (!(scale > 0.f) || !(scale < 1e30f)) return SE_ERR_SHAPE;
  const size_t need = snapkv_ws_bytes(*c, prompt_len, window);
  if (!ws || ws_bytes < need) return SE_ERR_WORKSPACE;
  SE_TRACE_CALL("snapkv_score_compact B=%d Hq=%d Hkv=%d L=%d W=%d pool=%d budget=%d", c->batch, c->n_q_heads,
                c->n_kv_heads, prompt_len, window, pool_kernel, budget);
  clear_stale_error();
  return launch_snapkv(*c, q_obs, k, v, prompt_len, window, pool_kernel, budget, scale, *out, k_out, v_out,
                       kept_pos, votes, out_seq_len, ws, stream);
}

se_status se_h2o_accumulate_evict(const se_cache* c, const float* logits, const float* lse,
                                  int32_t logit_cap, const int32_t* seq_len, int32_t* slot_pos,
                                  float* acc, int32_t cur_pos, int32_t heavy_budget,
                                  int32_t recent_window, int32_t* evict_slot, hipStream_t stream) {
  se_status st = check_cache(c);
  if (st != SE_OK) return st;
  if (!logits || !lse || !seq_len || !slot_pos || !acc || !evict_slot) return SE_ERR_NULL;
  if (logit_cap <= 0 || logit_cap < c->capacity) return SE_ERR_SHAPE;
  if (heavy_budget < 0 || recent_window < 0) return SE_ERR_BUDGET;
  if (int64_t(heavy_budget) + recent_window + 1 > c->capacity) return SE_ERR_BUDGET;
  if (cur_pos < 0) return SE_ERR_SHAPE;
  SE_TRACE_CALL("h2o_accumulate_evict B=%d Hq=%d Hkv=%d cap=%d pos=%d heavy=%d recent=%d", c->batch,
                c->n_q_heads, c->n_kv_heads, c->capacity, cur_pos, heavy_budget, recent_window);
  clear_stale_error();
  return launch_h2o(*c, logits, lse, logit_cap, seq_len, slot_pos, acc, cur_pos, heavy_budget, recent_window,
                    evict_slot, stream);
}

se_status se_h2o_decode_step(const se_cache* c, const void* q, void* k, void* v, const void* k_new,
                             const void* v_new, const int32_t* slot_in, int32_t* seq_len, int32_t* slot_pos,
                             float* acc, int32_t cur_pos, int32_t heavy_budget, int32_t recent_window, float scale,
                             float* out, float* lse, int32_t* evict_out, void* ws, size_t ws_bytes,
                             hipStream_t stream) {
  se_status st = check_cache(c);
  if (st != SE_OK) return st;
  if (!q || !k || !k_new || !seq_len || !slot_pos || !acc || !out || !evict_out || !ws ||
      (!c->latent && (!v || !v_new)))
    return SE_ERR_NULL;
  if (!aligned16(q) || !aligned16(k) || !aligned16(k_new) || !aligned16(out) || !aligned16(ws) ||
      (!c->latent && (!aligned16(v) || !aligned16(v_new))))
    return SE_ERR_ALIGN;
  if (slot_in != nullptr && slot_in == evict_out) return SE_ERR_SHAPE;   // read by every block of a row
  if (heavy_budget < 0 || recent_window < 0) return SE_ERR_BUDGET;
  if (int64_t(heavy_budget) + recent_window + 1 > c->capacity) return SE_ERR_BUDGET;
  if (cur_pos < 0) return SE_ERR_SHAPE;
  if (!(scale > 0.f) || !(scale < 1e30f)) return SE_ERR_SHAPE;
  if (int64_t(c->n_q_heads / c->n_kv_heads) * c->capacity > INT32_MAX) return SE_ERR_SHAPE;
  if (ws_bytes < h2o_step_ws_bytes(*c)) return SE_ERR_WORKSPACE;
  SE_TRACE_CALL("h2o_decode_step B=%d Hq=%d Hkv=%d cap=%d pos=%d heavy=%d recent=%d", c->batch, c->n_q_heads,
                c->n_kv_heads, c->capacity, cur_pos, heavy_budget, recent_window);
  clear_stale_error();
  return launch_h2o_step(*c, q, k, v, k_new, v_new, slot_in, seq_len, slot_pos, acc, cur_pos, heavy_budget,
                         recent_window, scale, out, lse, evict_out, ws, stream);
}

se_status se_h2o_prefill_init(const se_cache* c, const void* q_prompt, const void* k, const void* v,
                              int32_t prompt_len, int32_t heavy_budget, int32_t recent_window, float scale,
                              const se_cache* slots, void* k_slots, void* v_slots, int32_t* slot_pos, float* acc,
                              float* scores, void* ws, size_t ws_bytes, hipStream_t stream) {
  se_status st = check_cache(c);
  if (st != SE_OK) return st;
  st = check_cache(slots);
  if (st != SE_OK) return st;
  if (!q_prompt || !k || !v || !k_slots || !v_slots || !slot_pos || !acc || !ws) return SE_ERR_NULL;
  if (!aligned16(q_prompt) || !aligned16(k) || !aligned16(v) || !aligned16(k_slots) || !aligned16(v_slots) ||
      !aligned16(ws))
    return SE_ERR_ALIGN;
  if (c->dtype != SE_BF16) return SE_ERR_DTYPE;
  if (c->latent || (c->d_k != 64 && c->d_k != 128) || c->n_q_heads / c->n_kv_heads > 16) return SE_ERR_UNSUPPORTED;
  if (slots->batch != c->batch || slots->n_q_heads != c->n_q_heads || slots->n_kv_heads != c->n_kv_heads ||
      slots->d_k != c->d_k || slots->d_v != c->d_v || slots->dtype != c->dtype || slots->latent != c->latent)
    return SE_ERR_SHAPE;
  if (prompt_len < 2 || prompt_len > c->capacity) return SE_ERR_SHAPE;
  if (int64_t(prompt_len) * (c->n_q_heads / c->n_kv_heads) > (int64_t(1) << 30)) return SE_ERR_SHAPE;   // query rows index in int
  if (recent_window < 1 || recent_window >= prompt_len || heavy_budget < 1 ||
      int64_t(heavy_budget) + recent_window + 1 > slots->capacity)
    return SE_ERR_BUDGET;
  if (!(scale > 0.f) || !(scale < 1e30f)) return SE_ERR_SHAPE;
  if (ws_bytes < h2o_prefill_ws_bytes(*c, prompt_len, recent_window)) return SE_ERR_WORKSPACE;
  SE_TRACE_CALL("h2o_prefill_init B=%d Hq=%d Hkv=%d d_k=%d L=%d heavy=%d recent=%d", c->batch, c->n_q_heads,
                c->n_kv_heads, c->d_k, prompt_len, heavy_budget, recent_window);
  clear_stale_error();
  return launch_h2o_prefill(*c, q_prompt, k, v, prompt_len, heavy_budget, recent_window, scale, *slots, k_slots,
                            v_slots, slot_pos, acc, scores, ws, stream);
}

se_status se_omnikv_topk(const se_cache* c, const float* logits, const float* lse, int32_t logit_cap,
                         const int32_t* seq_len, int32_t top_k, int32_t* view_idx,
                         int32_t* view_len, float* scores, void* ws, size_t ws_bytes,
                         hipStream_t stream) {
  se_status st = check_cache(c);
  if (st != SE_OK) return st;
  if (!logits || !lse || !seq_len || !view_idx || !view_len) return SE_ERR_NULL;
  if (logit_cap <= 0) return SE_ERR_SHAPE;
  if (top_k < 1 || top_k > logit_cap) return SE_ERR_BUDGET;
  const size_t need = scores ? 0 : omnikv_ws_bytes(*c, logit_cap, top_k);
  if (need > 0 && (!ws || ws_bytes < need)) return SE_ERR_WORKSPACE;
  SE_TRACE_CALL("omnikv_topk B=%d Hq=%d Hkv=%d cap=%d k=%d", c->batch, c->n_q_heads, c->n_kv_heads, logit_cap,
                top_k);
  clear_stale_error();
  return launch_omnikv(*c, logits, lse, logit_cap, seq_len, top_k, view_idx, view_len, scores, ws, stream);
}

}  // extern "C"
