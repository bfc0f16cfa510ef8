// KV append and Quest page metadata (per-page elementwise min / max of K).
//
// The per-page summary index of dynamic-sparse methods (tokendh.com explainer,
// section "历史太长,会撑爆什么") is realised as the min and max of every key
// dimension over the page's valid tokens.  min / max of stored values is exact,
// so the metadata keeps K's element type.
#include "se_internal.hpp"

namespace se {

// Zero fill of a workspace: 16-byte stores, then the trailing bytes.
__global__ __launch_bounds__(256) void zero_fill_kernel(uint4* __restrict__ p, size_t n16, uint8_t* __restrict__ tail,
                                                        int ntail) {
  const size_t stride = size_t(gridDim.x) * blockDim.x;
  for (size_t i = size_t(blockIdx.x) * blockDim.x + threadIdx.x; i < n16; i += stride) p[i] = make_uint4(0, 0, 0, 0);
  if (blockIdx.x == 0 && int(threadIdx.x) < ntail) tail[threadIdx.x] = 0;
}

se_status launch_zero_fill(void* p, size_t bytes, hipStream_t s) {
  const size_t n16 = bytes / 16;
  const int ntail = int(bytes - n16 * 16);
  const int grid = int(std::max<size_t>(1, std::min<size_t>(1024, (n16 + 255) / 256)));
  hipLaunchKernelGGL(zero_fill_kernel, dim3(grid), dim3(256), 0, s, (uint4*)p, n16, (uint8_t*)p + n16 * 16, ntail);
  return launch_status();
}

// One block per batch row: copies the new row of every KV head, then bumps seq_len.
__global__ __launch_bounds__(256) void kv_append_kernel(
    uint32_t* __restrict__ k, uint32_t* __restrict__ v, const uint32_t* __restrict__ k_new,
    const uint32_t* __restrict__ v_new, const int32_t* __restrict__ slot, int32_t* __restrict__ seq_len,
    int Hkv, int cap, int kwords, int vwords) {
  const int b = blockIdx.x;
  const int len = seq_len[b];
  const bool bump = slot == nullptr || slot[b * Hkv] < 0;
  for (int h = 0; h < Hkv; ++h) {
    int pos = len;
    if (slot != nullptr && slot[b * Hkv + h] >= 0) pos = slot[b * Hkv + h];
    if (pos < 0 || pos >= cap) continue;
    const size_t unit = size_t(b) * Hkv + h;
    uint32_t* kd = k + (unit * cap + pos) * kwords;
    const uint32_t* ks = k_new + unit * kwords;
    for (int i = threadIdx.x; i < kwords; i += blockDim.x) kd[i] = ks[i];
    if (v != nullptr) {
      uint32_t* vd = v + (unit * cap + pos) * vwords;
      const uint32_t* vs = v_new + unit * vwords;
      for (int i = threadIdx.x; i < vwords; i += blockDim.x) vd[i] = vs[i];
    }
  }
  __syncthreads();
  if (threadIdx.x == 0 && bump && len < cap) seq_len[b] = len + 1;
}

se_status launch_kv_append(const se_cache& c, void* k, void* v, const void* k_new, const void* v_new,
                           const int32_t* slot, int32_t* seq_len, hipStream_t s) {
  const int esz = c.dtype == SE_F32 ? 4 : 2;
  const int kwords = c.d_k * esz / 4, vwords = c.d_v * esz / 4;
  hipLaunchKernelGGL(kv_append_kernel, dim3(c.batch), dim3(256), 0, s, (uint32_t*)k,
                     c.latent ? nullptr : (uint32_t*)v, (const uint32_t*)k_new,
                     c.latent ? nullptr : (const uint32_t*)v_new, slot, seq_len, c.n_kv_heads,
                     c.capacity, kwords, vwords);
  return launch_status();
}

// ------------------------------------------------------------------ page metadata

template <typename T> __device__ __forceinline__ T from_f32(float x);
template <> __device__ __forceinline__ float from_f32<float>(float x) { return x; }
template <> __device__ __forceinline__ bf16_t from_f32<bf16_t>(float x) {
  return bf16_t{uint16_t(__float_as_uint(x) >> 16)};  // exact: x is a stored bf16 value
}

// grid: (page slots, units).  first_page < 0: one page per unit, the one holding
// slot seq_len - 1.  Otherwise page first_page + blockIdx.x (+ gridDim.x * i).
template <typename T>
__global__ __launch_bounds__(256) void page_meta_kernel(
    const T* __restrict__ k, T* __restrict__ kmin, T* __restrict__ kmax, const int32_t* __restrict__ seq_len,
    int Hkv, int cap, int D, int P, int first_page) {
  const int unit = blockIdx.y;
  const int b = unit / Hkv;
  const int len = min(seq_len[b], cap);
  const int npages = (len + P - 1) / P;
  const int n_cap_pages = (cap + P - 1) / P;
  const T* ku = k + size_t(unit) * cap * D;
  int p0, pstep;
  if (first_page < 0) {
    if (blockIdx.x != 0 || len <= 0) return;
    p0 = (len - 1) / P;
    pstep = npages;  // single page
  } else {
    p0 = first_page + blockIdx.x;
    pstep = gridDim.x;
  }
  for (int p = p0; p < npages && p < n_cap_pages; p += pstep) {
    const int t0 = p * P, t1 = min(len, t0 + P);
    for (int d = threadIdx.x; d < D; d += blockDim.x) {
      float mn = INFINITY, mx = -INFINITY;
      for (int t = t0; t < t1; ++t) {
        float x = to_f32(ku[size_t(t) * D + d]);
        mn = fminf(mn, x);
        mx = fmaxf(mx, x);
      }
      const size_t o = (size_t(unit) * n_cap_pages + p) * D + d;
      kmin[o] = from_f32<T>(mn);
      kmax[o] = from_f32<T>(mx);
    }
    if (first_page < 0) break;
  }
}

// ------------------------------------------------------------------ append + metadata in one launch
// One block per batch row: writes the new row of every KV head (as
// kv_append_kernel), then rebuilds the min / max of the page holding each
// written slot over the slots below the new length, then bumps seq_len.  Works
// on 32-bit words: a bf16 word holds two dimensions, min / max taken on each.
template <bool BF16>
__global__ __launch_bounds__(256) void kv_append_meta_kernel(
    uint32_t* __restrict__ k, uint32_t* __restrict__ v, const uint32_t* __restrict__ k_new,
    const uint32_t* __restrict__ v_new, const int32_t* __restrict__ slot, int32_t* __restrict__ seq_len,
    uint32_t* __restrict__ kmin, uint32_t* __restrict__ kmax, int Hkv, int cap, int kwords, int vwords, int P) {
  const int b = blockIdx.x;
  const int len = seq_len[b];
  const bool bump = slot == nullptr || slot[b * Hkv] < 0;
  const int new_len = (bump && len < cap) ? len + 1 : len;
  const int n_cap_pages = (cap + P - 1) / P;
  auto slot_of = [&](int h) { return (slot != nullptr && slot[b * Hkv + h] >= 0) ? slot[b * Hkv + h] : len; };
  for (int i = threadIdx.x; i < Hkv * kwords; i += blockDim.x) {
    const int h = i / kwords, wd = i - h * kwords, pos = slot_of(h);
    if (pos < 0 || pos >= cap) continue;
    const size_t unit = size_t(b) * Hkv + h;
    k[(unit * cap + pos) * kwords + wd] = k_new[unit * kwords + wd];
  }
  if (v != nullptr)
    for (int i = threadIdx.x; i < Hkv * vwords; i += blockDim.x) {
      const int h = i / vwords, wd = i - h * vwords, pos = slot_of(h);
      if (pos < 0 || pos >= cap) continue;
      const size_t unit = size_t(b) * Hkv + h;
      v[(unit * cap + pos) * vwords + wd] = v_new[unit * vwords + wd];
    }
  __syncthreads();   // the block's row writes are visible to its page reads
  for (int i = threadIdx.x; i < Hkv * kwords; i += blockDim.x) {
    const int h = i / kwords, wd = i - h * kwords, pos = slot_of(h);
    if (pos < 0 || pos >= cap) continue;
    const int page = pos / P, t0 = page * P, t1 = min(new_len, t0 + P);
    if (t0 >= t1) continue;
    const size_t unit = size_t(b) * Hkv + h;
    const uint32_t* col = k + unit * cap * kwords + wd;
    float mn0 = INFINITY, mx0 = -INFINITY, mn1 = INFINITY, mx1 = -INFINITY;
#pragma unroll 4
    for (int t = t0; t < t1; ++t) {
      const uint32_t x = col[size_t(t) * kwords];
      if (BF16) {
        const float lo = bf16_lo(x), hi = bf16_hi(x);
        mn0 = fminf(mn0, lo); mx0 = fmaxf(mx0, lo);
        mn1 = fminf(mn1, hi); mx1 = fmaxf(mx1, hi);
      } else {
        const float f = __uint_as_float(x);
        mn0 = fminf(mn0, f); mx0 = fmaxf(mx0, f);
      }
    }
    const size_t o = (unit * n_cap_pages + page) * kwords + wd;
    if (BF16) {   // exact: every value is a stored bf16
      kmin[o] = (__float_as_uint(mn0) >> 16) | (__float_as_uint(mn1) & 0xffff0000u);
      kmax[o] = (__float_as_uint(mx0) >> 16) | (__float_as_uint(mx1) & 0xffff0000u);
    } else {
      kmin[o] = __float_as_uint(mn0);
      kmax[o] = __float_as_uint(mx0);
    }
  }
  __syncthreads();
  if (threadIdx.x == 0 && new_len != len) seq_len[b] = new_len;
}

se_status launch_kv_append_meta(const se_cache& c, void* k, void* v, const void* k_new, const void* v_new,
                                const int32_t* slot, int32_t* seq_len, void* kmin, void* kmax, int page_size,
                                hipStream_t s) {
  const int esz = c.dtype == SE_F32 ? 4 : 2;
  const int kwords = c.d_k * esz / 4, vwords = c.d_v * esz / 4;
  void* vv = c.latent ? nullptr : v;
  const void* vn = c.latent ? nullptr : v_new;
  if (c.dtype == SE_F32)
    hipLaunchKernelGGL(kv_append_meta_kernel<false>, dim3(c.batch), dim3(256), 0, s, (uint32_t*)k, (uint32_t*)vv,
                       (const uint32_t*)k_new, (const uint32_t*)vn, slot, seq_len, (uint32_t*)kmin,
                       (uint32_t*)kmax, c.n_kv_heads, c.capacity, kwords, vwords, page_size);
  else
    hipLaunchKernelGGL(kv_append_meta_kernel<true>, dim3(c.batch), dim3(256), 0, s, (uint32_t*)k, (uint32_t*)vv,
                       (const uint32_t*)k_new, (const uint32_t*)vn, slot, seq_len, (uint32_t*)kmin,
                       (uint32_t*)kmax, c.n_kv_heads, c.capacity, kwords, vwords, page_size);
  return launch_status();
}

se_status launch_page_meta(const se_cache& c, const void* k, void* kmin, void* kmax,
                           const int32_t* seq_len, int page_size, int first_page, hipStream_t s) {
  const int units = c.batch * c.n_kv_heads;
  const int n_cap_pages = ceil_div(c.capacity, page_size);
  dim3 grid(first_page < 0 ? 1 : std::min(n_cap_pages, 4096), units);
  if (c.dtype == SE_F32)
    hipLaunchKernelGGL(page_meta_kernel<float>, grid, dim3(256), 0, s, (const float*)k, (float*)kmin,
                       (float*)kmax, seq_len, c.n_kv_heads, c.capacity, c.d_k, page_size, first_page);
  else
    hipLaunchKernelGGL(page_meta_kernel<bf16_t>, grid, dim3(256), 0, s, (const bf16_t*)k, (bf16_t*)kmin,
                       (bf16_t*)kmax, seq_len, c.n_kv_heads, c.capacity, c.d_k, page_size, first_page);
  return launch_status();
}

}  // namespace se
