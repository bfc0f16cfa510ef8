// FP8 KV rows: OCP E4M3 codes with one power-of-two scale per row.
//
// tokendh.com explainer, section "历史太长,会撑爆什么": KV quantization keeps the
// history at lower precision together with what is needed to restore it.  Here a
// stored row (one token of one KV head) is d_k E4M3 codes plus one byte
// s = e + 127 (E8M0): the row's values are code * 2^e, with e the smallest
// exponent >= -126 for which the row's largest magnitude times 2^-e is at most
// 448, and every code the nearest E4M3 value of x * 2^-e, ties to the even code.
// Those stored values are exact in bf16, so page metadata, selection and
// attention over an FP8 cache are the bf16 path over the stored values.
#include "fp8_row.hpp"
#include "mfma_util.hpp"

namespace se {

// grid: (row groups, units); TPR = d / 8 threads per row, 256 / TPR rows per block.
// Rows [0, seq_len[b]) of K and V (bf16) -> codes and scale bytes.
template <int D>
__global__ __launch_bounds__(256) void fp8_quantize_kernel(const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
                                                           const int32_t* __restrict__ seq_len,
                                                           uint8_t* __restrict__ kq, uint8_t* __restrict__ vq,
                                                           uint8_t* __restrict__ ks, uint8_t* __restrict__ vs,
                                                           int Hkv, int cap) {
  constexpr int TPR = D / 8, RPB = 256 / TPR;
  const int unit = blockIdx.y, b = unit / Hkv;
  const int len = min(max(seq_len[b], 0), cap);
  const int row = blockIdx.x * RPB + threadIdx.x / TPR, part = threadIdx.x % TPR;
  if (blockIdx.x * RPB >= len) return;       // whole block past the history (rows of a block are contiguous)
  const bool ok = row < len;
  const size_t r = size_t(unit) * cap + (ok ? row : 0);
#pragma unroll
  for (int which = 0; which < 2; ++which) {
    const uint16_t* src = which ? v : k;
    uint8_t* dq = which ? vq : kq;
    uint8_t* ds = which ? vs : ks;
    int e;
    const uint2 c = fp8_quantize8<TPR>(ld16(src + r * D + 8 * part), e);
    if (ok) {
      *reinterpret_cast<uint2*>(dq + r * D + 8 * part) = c;
      if (part == 0) ds[r] = uint8_t(e + 127);
    }
  }
}

// grid: (page slots, units).  Min / max of the stored K values of each page, in
// row order from +-inf (the order every metadata kernel here uses).
template <int D>
__global__ __launch_bounds__(256) void fp8_page_meta_kernel(const uint8_t* __restrict__ kq, const uint8_t* __restrict__ ks,
                                                            const int32_t* __restrict__ seq_len, uint16_t* __restrict__ kmin,
                                                            uint16_t* __restrict__ kmax, int Hkv, int cap, int P) {
  const int unit = blockIdx.y, b = unit / Hkv;
  const int len = min(max(seq_len[b], 0), cap);
  const int npages = (len + P - 1) / P, ncp = (cap + P - 1) / P;
  for (int p = blockIdx.x; p < npages; p += gridDim.x) {
    const int t0 = p * P, t1 = min(len, t0 + P);
    for (int d = threadIdx.x; d < D; d += blockDim.x) {
      float mn = INFINITY, mx = -INFINITY;
      for (int t = t0; t < t1; ++t) {
        const size_t r = size_t(unit) * cap + t;
        const float x = fp8_value<0>(kq[r * D + d], int(ks[r]) - 127);
        mn = fminf(mn, x);
        mx = fmaxf(mx, x);
      }
      const size_t o = (size_t(unit) * ncp + p) * D + d;
      kmin[o] = uint16_t(__float_as_uint(mn) >> 16);   // exact: stored values are bf16 values
      kmax[o] = uint16_t(__float_as_uint(mx) >> 16);
    }
  }
}

// One block per batch row: quantizes the new K / V row of every KV head into slot
// seq_len[b], folds the new row's stored K values into the min / max of its page
// (the row alone on a fresh page; kmin / kmax hold the page's in-order min / max,
// so fminf(old, new) is the last step of the rebuild), then bumps seq_len.
template <int D>
__global__ __launch_bounds__(256) void fp8_append_kernel(uint8_t* __restrict__ kq, uint8_t* __restrict__ vq,
                                                         uint8_t* __restrict__ ks, uint8_t* __restrict__ vs,
                                                         const uint16_t* __restrict__ k_new,
                                                         const uint16_t* __restrict__ v_new, int32_t* __restrict__ seq_len,
                                                         uint16_t* __restrict__ kmin, uint16_t* __restrict__ kmax,
                                                         int Hkv, int cap, int P) {
  constexpr int TPR = D / 8;
  const int b = blockIdx.x;
  const int len = seq_len[b];
  if (len < 0 || len >= cap) return;         // no room: nothing written
  const int ncp = (cap + P - 1) / P;
  const bool fresh = len % P == 0;
  // rows: (head, K or V) pairs, TPR threads each
  for (int i = threadIdx.x; i < Hkv * 2 * TPR; i += blockDim.x) {
    const int part = i % TPR, rw = i / TPR, h = rw >> 1, isv = rw & 1;
    const size_t unit = size_t(b) * Hkv + h, r = unit * cap + len;
    int e;
    const uint2 c = fp8_quantize8<TPR>(ld16((isv ? v_new : k_new) + unit * D + 8 * part), e);
    *reinterpret_cast<uint2*>((isv ? vq : kq) + r * D + 8 * part) = c;
    if (part == 0) (isv ? vs : ks)[r] = uint8_t(e + 127);
    if (!isv && kmin != nullptr) {
      const size_t mo = (unit * ncp + len / P) * D + 8 * part;
      const u32x4 omn = ld16(kmin + mo), omx = ld16(kmax + mo);
      u32x4 nmn, nmx;
#pragma unroll
      for (int j = 0; j < 4; ++j) {   // bf16 pair j = codes 2j, 2j + 1
        const uint32_t w = j < 2 ? c.x : c.y;
        const float lo = (j & 1) ? fp8_value<2>(w, e) : fp8_value<0>(w, e);
        const float hi = (j & 1) ? fp8_value<3>(w, e) : fp8_value<1>(w, e);
        const float mnl = fminf(fresh ? INFINITY : bf16_lo(omn[j]), lo), mnh = fminf(fresh ? INFINITY : bf16_hi(omn[j]), hi);
        const float mxl = fmaxf(fresh ? -INFINITY : bf16_lo(omx[j]), lo), mxh = fmaxf(fresh ? -INFINITY : bf16_hi(omx[j]), hi);
        nmn[j] = (__float_as_uint(mnl) >> 16) | (__float_as_uint(mnh) & 0xffff0000u);
        nmx[j] = (__float_as_uint(mxl) >> 16) | (__float_as_uint(mxh) & 0xffff0000u);
      }
      *reinterpret_cast<u32x4*>(kmin + mo) = nmn;
      *reinterpret_cast<u32x4*>(kmax + mo) = nmx;
    }
  }
  __syncthreads();
  if (threadIdx.x == 0) seq_len[b] = len + 1;
}

se_status launch_fp8_quantize(const se_cache& c, const void* k, const void* v, const int32_t* seq_len, void* kq,
                              void* vq, void* ks, void* vs, void* kmin, void* kmax, int page_size, hipStream_t s) {
  const int units = c.batch * c.n_kv_heads;
#define SE_Q(DD)                                                                                                     \
  hipLaunchKernelGGL(fp8_quantize_kernel<DD>, dim3(ceil_div(c.capacity, 256 / (DD / 8)), units), dim3(256), 0, s,    \
                     (const uint16_t*)k, (const uint16_t*)v, seq_len, (uint8_t*)kq, (uint8_t*)vq, (uint8_t*)ks,     \
                     (uint8_t*)vs, c.n_kv_heads, c.capacity);                                                        \
  if (kmin != nullptr)                                                                                               \
    hipLaunchKernelGGL(fp8_page_meta_kernel<DD>, dim3(std::min(ceil_div(c.capacity, page_size), 4096), units),      \
                       dim3(DD), 0, s, (const uint8_t*)kq, (const uint8_t*)ks, seq_len, (uint16_t*)kmin,             \
                       (uint16_t*)kmax, c.n_kv_heads, c.capacity, page_size)
  if (c.d_k == 128) { SE_Q(128); } else { SE_Q(64); }
#undef SE_Q
  return launch_status();
}

se_status launch_fp8_append(const se_cache& c, void* kq, void* vq, void* ks, void* vs, const void* k_new,
                            const void* v_new, int32_t* seq_len, void* kmin, void* kmax, int page_size, hipStream_t s) {
#define SE_A(DD)                                                                                                   \
  hipLaunchKernelGGL(fp8_append_kernel<DD>, dim3(c.batch), dim3(256), 0, s, (uint8_t*)kq, (uint8_t*)vq,             \
                     (uint8_t*)ks, (uint8_t*)vs, (const uint16_t*)k_new, (const uint16_t*)v_new, seq_len,           \
                     (uint16_t*)kmin, (uint16_t*)kmax, c.n_kv_heads, c.capacity, page_size)
  if (c.d_k == 128) SE_A(128); else SE_A(64);
#undef SE_A
  return launch_status();
}

}  // namespace se
