// Internal declarations and device helpers of libse (gfx950, wave64).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <math.h>
#include <algorithm>
#include "../../include/se.h"

namespace se {

constexpr int WAVE = 64;

// ------------------------------------------------------------------ element access
struct bf16_t { uint16_t bits; };

__device__ __forceinline__ float to_f32(float x) { return x; }
__device__ __forceinline__ float to_f32(bf16_t x) { return __uint_as_float(uint32_t(x.bits) << 16); }
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// Round-to-nearest-even fp32 -> bf16 (finite inputs).
__device__ __forceinline__ uint16_t f32_to_bf16_bits(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7fffu + ((u >> 16) & 1u);
  return uint16_t(u >> 16);
}

// ------------------------------------------------------------------ selection keys
// Total order on floats as unsigned ints (larger float -> larger key); -0.0 is
// canonicalised to +0.0 first so that the two zeros tie.
__device__ __forceinline__ uint32_t ordered_bits(float x) {
  uint32_t u = __float_as_uint(x + 0.0f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
// Unique key: larger score first, then lower index.
__device__ __forceinline__ uint64_t key_desc_score_asc_index(float s, uint32_t idx) {
  return (uint64_t(ordered_bits(s)) << 32) | uint64_t(0xffffffffu - idx);
}

// ------------------------------------------------------------------ wave / block helpers
__device__ __forceinline__ float wave_max(float v) {
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, WAVE));
  return v;
}
__device__ __forceinline__ float wave_sum(float v) {
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, WAVE);
  return v;
}
__device__ __forceinline__ int wave_sum_i(int v) {
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, WAVE);
  return v;
}
// Inclusive prefix sum across the wave.
__device__ __forceinline__ int wave_incl_scan(int v) {
  const int lane = threadIdx.x & (WAVE - 1);
  for (int o = 1; o < WAVE; o <<= 1) {
    int t = __shfl_up(v, o, WAVE);
    if (lane >= o) v += t;
  }
  return v;
}

// Exclusive prefix sum over the block; `tmp` is >= BLOCK/64 ints of LDS.  Also returns the total.
template <int BLOCK>
__device__ __forceinline__ int block_excl_scan(int v, int* tmp, int* total) {
  const int lane = threadIdx.x & (WAVE - 1), w = threadIdx.x / WAVE;
  int inc = wave_incl_scan(v);
  if (lane == WAVE - 1) tmp[w] = inc;
  __syncthreads();
  int base = 0, tot = 0;
  for (int i = 0; i < BLOCK / WAVE; ++i) {
    int t = tmp[i];
    if (i < w) base += t;
    tot += t;
  }
  __syncthreads();
  *total = tot;
  return base + inc - v;
}

// ------------------------------------------------------------------ block top-k
// Exact top-k by unique 64-bit key, then an order-preserving compaction: the
// chosen indices come out in ascending index order.  `score(i)` gives the float
// score of candidate i < n; ties go to the lower index.  Writes out[0..min(k,n))
// and pads out[.. k) with -1.
//
// Radix select: the bits every candidate shares are skipped (one OR / AND
// reduction), then 8-bit digits are resolved most significant first.  The
// digit histogram is kept in 8 LDS copies (one per thread % 8) so that a skewed
// digit does not serialise the atomics; the search stops as soon as one digit
// bucket holds exactly the keys still to choose.
constexpr int TOPK_HCOPIES = 8;
struct TopkShared {
  uint32_t hist[TOPK_HCOPIES][256];
  uint64_t red_or[16], red_and[16];
  int digit, rem, cnt;
  int scan_tmp[16];
};

template <int BLOCK, class ScoreFn>
__device__ int block_topk_ascending(ScoreFn score, int n, int k, int32_t* out, TopkShared& sh) {
  constexpr int NW = BLOCK / WAVE;
  const int tid = threadIdx.x, lane = tid & (WAVE - 1), w = tid / WAVE;
  const int kk = k < n ? k : n;
  // contiguous candidate range of this thread (keeps the compaction order-preserving)
  const int per = (n + BLOCK - 1) / BLOCK;
  const int lo = min(n, tid * per), hi = min(n, lo + per);
  uint64_t threshold = 0;  // select keys >= threshold
  if (kk > 0 && kk < n) {
    uint64_t kor = 0, kand = ~0ull;
    for (int i = lo; i < hi; ++i) {
      const uint64_t key = key_desc_score_asc_index(score(i), uint32_t(i));
      kor |= key;
      kand &= key;
    }
    for (int o = WAVE / 2; o > 0; o >>= 1) {
      kor |= __shfl_xor(kor, o, WAVE);
      kand &= __shfl_xor(kand, o, WAVE);
    }
    if (lane == 0) { sh.red_or[w] = kor; sh.red_and[w] = kand; }
    __syncthreads();
    kor = 0; kand = ~0ull;
    for (int i = 0; i < NW; ++i) { kor |= sh.red_or[i]; kand &= sh.red_and[i]; }
    const int top = 63 - __clzll((long long)(kor ^ kand));   // highest differing bit (keys are unique)
    uint64_t mask = top == 63 ? 0ull : (~0ull << (top + 1));
    uint64_t prefix = kand & mask;
    int remaining = kk;
    const int cp = tid & (TOPK_HCOPIES - 1);
    for (int hb = top; hb >= 0; hb -= 8) {
      const int shift = hb >= 7 ? hb - 7 : 0;
      const uint32_t dmask = (1u << (hb - shift + 1)) - 1u;
      for (int j = tid; j < TOPK_HCOPIES * 256; j += BLOCK) (&sh.hist[0][0])[j] = 0;
      __syncthreads();
      for (int i = lo; i < hi; ++i) {
        const uint64_t key = key_desc_score_asc_index(score(i), uint32_t(i));
        if ((key & mask) == prefix) atomicAdd(&sh.hist[cp][uint32_t(key >> shift) & dmask], 1u);
      }
      __syncthreads();
      if (tid < WAVE) {
        // lane owns digits 4*lane .. 4*lane+3
        int c4[4], own = 0;
        for (int j = 0; j < 4; ++j) {
          int s = 0;
          for (int c = 0; c < TOPK_HCOPIES; ++c) s += int(sh.hist[c][4 * tid + j]);
          c4[j] = s;
          own += s;
        }
        int incl = own;   // keys whose digit lies in this lane's block or above
        for (int o = 1; o < WAVE; o <<= 1) {
          const int t = __shfl_down(incl, o, WAVE);
          if (tid + o < WAVE) incl += t;
        }
        const int above = incl - own;
        if (above < remaining && remaining <= incl) {
          int acc = above;
          for (int j = 3; j >= 0; --j) {
            if (acc + c4[j] >= remaining) {
              sh.digit = 4 * tid + j;
              sh.rem = remaining - acc;
              sh.cnt = c4[j];
              break;
            }
            acc += c4[j];
          }
        }
      }
      __syncthreads();
      const int fd = sh.digit, frem = sh.rem, fcnt = sh.cnt;
      __syncthreads();
      prefix |= uint64_t(uint32_t(fd)) << shift;
      mask |= uint64_t(dmask) << shift;
      remaining = frem;
      if (fcnt == frem) break;   // the whole digit bucket is selected
    }
    threshold = prefix;
  }
  int cnt = 0;
  if (kk > 0)
    for (int i = lo; i < hi; ++i) cnt += key_desc_score_asc_index(score(i), uint32_t(i)) >= threshold;
  int total;
  int off = block_excl_scan<BLOCK>(cnt, sh.scan_tmp, &total);
  if (kk > 0)
    for (int i = lo; i < hi; ++i)
      if (key_desc_score_asc_index(score(i), uint32_t(i)) >= threshold) {
        if (off < k) out[off] = i;
        ++off;
      }
  for (int i = kk + tid; i < k; i += BLOCK) out[i] = -1;
  return kk;
}


// ------------------------------------------------------------------ launch helpers
inline se_status launch_status() {
  return hipGetLastError() == hipSuccess ? SE_OK : SE_ERR_HIP;
}
inline int ceil_div(int a, int b) { return (a + b - 1) / b; }

// ------------------------------------------------------------------ launchers (host)
se_status launch_zero_fill(void* p, size_t bytes, hipStream_t s);
se_status launch_kv_append(const se_cache& c, void* k, void* v, const void* k_new, const void* v_new,
                           const int32_t* slot, int32_t* seq_len, hipStream_t s);
se_status launch_page_meta(const se_cache& c, const void* k, void* kmin, void* kmax,
                           const int32_t* seq_len, int page_size, int first_page, hipStream_t s);
size_t quest_ws_bytes(const se_cache& c, int page_size, int top_pages);
se_status launch_quest(const se_cache& c, const void* q, const void* kmin, const void* kmax,
                       const int32_t* seq_len, int page_size, int top_pages, int32_t* view_idx,
                       int32_t* view_len, float* page_score, void* ws, hipStream_t s);
int attn_auto_splits(const se_cache& c, int slots);
size_t attn_ws_bytes(const se_cache& c, int slots, int num_splits);
se_status launch_attn(const se_cache& c, const void* q, const void* k, const void* v,
                      const int32_t* seq_len, const int32_t* view_idx, const int32_t* view_len,
                      int view_cap, int granularity, float scale, float* out, float* lse,
                      float* logits, int logit_cap, int num_splits, void* ws, hipStream_t s);
size_t snapkv_ws_bytes(const se_cache& c, int prompt_len, int window);
se_status launch_snapkv(const se_cache& c, const void* q_obs, const void* k, const void* v,
                        int prompt_len, int window, int pool_kernel, int budget, float scale,
                        const se_cache& out, void* k_out, void* v_out, int32_t* kept_pos,
                        float* votes, int32_t* out_seq_len, void* ws, hipStream_t s);
se_status launch_h2o(const se_cache& c, const float* logits, const float* lse, int logit_cap,
                     const int32_t* seq_len, int32_t* slot_pos, float* acc, int cur_pos, int heavy,
                     int recent, int32_t* evict_slot, hipStream_t s);
size_t omnikv_ws_bytes(const se_cache& c, int logit_cap, int top_k);
se_status launch_omnikv(const se_cache& c, const float* logits, const float* lse, int logit_cap,
                        const int32_t* seq_len, int top_k, int32_t* view_idx, int32_t* view_len,
                        float* scores, void* ws, hipStream_t s);

}  // namespace se
