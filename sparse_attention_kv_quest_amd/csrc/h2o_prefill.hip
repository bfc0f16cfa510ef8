// H2O scores at the end of a prefill: how much attention every prompt key got.
//
// tokendh.com explainer, sections "历史太长,会撑爆什么" and "把边界划在'生命周期'上":
// H2O keeps a continuously accumulated table of the attention each token
// receives and evicts by it.  At the end of the prefill that table is the
// attention of every prompt query: acc0[j] = sum over the group's heads and the
// queries i >= j of softmax_i(scale q_i . k)[j] (causal).  Two MFMA passes over
// the causal half of the (query, key) square:
//   A: per (head, query) row, the log2-sum-exp2 of sc2 * q . k over keys <= i;
//   B: per key, the sum of exp2(sc2 * q . k - lse2) over the later queries.
// Both use S^T[key][head] = K . Q^T with the group's heads (G <= 16) in the MFMA
// N dimension: A = 16 key rows (lane: key c16, dims 32c + 8g ..), B = one
// position's queries (lane: head c16, the same dims).  K tiles (pass A) and Q
// tiles (pass B) go through double-buffered LDS shared by the block's 8 waves.
// The kept set then follows the SnapKV keep rule on acc0 (no pooling).
#include "se_internal.hpp"
#include "mfma_util.hpp"

namespace se {

constexpr int HP_WAVES = 8;
constexpr int HP_PPW = 8;                       // pass A: query positions per wave
constexpr int HP_POS = HP_WAVES * HP_PPW;       // pass A: 64 positions per block
constexpr int HP_KT = 32;                       // pass A: keys per K tile
constexpr int HP_KB = 4;                        // pass B: 16-key blocks per wave
constexpr int HP_KEYS = HP_WAVES * HP_KB * 16;  // pass B: 512 keys per block
constexpr int HP_QT = 8;                        // pass B: positions per Q tile

struct HpArgs {
  const uint16_t* q;    // [B][Hq][L][D] every prompt query
  const uint16_t* k;    // [B][Hkv][cap][D]
  float* lse2;          // [units][G][L]
  float* acc0;          // [units][L]
  float* votes;         // [units][L - recent]: acc0 of the candidates of the keep rule
  int Hq, Hkv, G, cap, L, n_cand;
  float sc2;            // scale * log2(e)
};

template <int D>
__global__ __launch_bounds__(512) void hp_rowlse_kernel(HpArgs a) {
  constexpr int NKS = D / 32, PITCH = D + 8, CH = D / 8;   // CH 16-byte chunks per row
  __shared__ __align__(16) uint16_t kt[2][HP_KT][PITCH];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, g = lane >> 4, c16 = lane & 15;
  const int unit = blockIdx.y, b = unit / a.Hkv, kvh = unit % a.Hkv;
  const int L = a.L, p_blk = blockIdx.x * HP_POS;
  if (p_blk >= L) return;                              // uniform per block
  const int p_w = p_blk + w * HP_PPW;
  const uint16_t* ku = a.k + size_t(unit) * a.cap * D;
  u32x4 qv[HP_PPW][NKS];
#pragma unroll
  for (int pp = 0; pp < HP_PPW; ++pp) {
    const bool ok = c16 < a.G && p_w + pp < L;
    const uint16_t* qp = a.q + ((size_t(b) * a.Hq + size_t(kvh) * a.G + (ok ? c16 : 0)) * L + (ok ? p_w + pp : 0)) * D;
#pragma unroll
    for (int c = 0; c < NKS; ++c) qv[pp][c] = ok ? ld16(qp + 8 * g + 32 * c) : u32x4{0, 0, 0, 0};
  }
  float m[HP_PPW], l[HP_PPW];
#pragma unroll
  for (int pp = 0; pp < HP_PPW; ++pp) { m[pp] = -INFINITY; l[pp] = 0.f; }
  const int ntiles = (min(L, p_blk + HP_POS) - 1) / HP_KT + 1;   // keys up to the block's last position
  // one 16-byte chunk of the tile per thread (threads past the tile idle)
  const int lk = threadIdx.x / CH, lc = threadIdx.x % CH;
  const bool loader = lk < HP_KT;
  auto fetch = [&](int t) -> u32x4 {
    const int key = min(t * HP_KT + lk, L - 1);
    return ld16(ku + size_t(key) * D + 8 * lc);
  };
  if (loader) *reinterpret_cast<u32x4*>(&kt[0][lk][8 * lc]) = fetch(0);
  __syncthreads();
  for (int t = 0; t < ntiles; ++t) {
    const int buf = t & 1;
    u32x4 nxt = {0, 0, 0, 0};
    if (loader && t + 1 < ntiles) nxt = fetch(t + 1);
#pragma unroll
    for (int hf = 0; hf < 2; ++hf) {
      u32x4 ak[NKS];
#pragma unroll
      for (int c = 0; c < NKS; ++c) ak[c] = *reinterpret_cast<const u32x4*>(&kt[buf][hf * 16 + c16][8 * g + 32 * c]);
      const int kbase = t * HP_KT + hf * 16 + 4 * g;
#pragma unroll
      for (int pp = 0; pp < HP_PPW; ++pp) {
        const int pos = p_w + pp;
        f32x4 s = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int c = 0; c < NKS; ++c) s = mfma_bf16_16x16x32(ak[c], qv[pp][c], s);
        float v[4], hm = -INFINITY;
#pragma unroll
        for (int ii = 0; ii < 4; ++ii) {
          v[ii] = kbase + ii <= pos ? s[ii] * a.sc2 : -INFINITY;   // causal (pos < L implies key < L)
          hm = fmaxf(hm, v[ii]);
        }
        hm = fmaxf(hm, __shfl_xor(hm, 16, 64));
        hm = fmaxf(hm, __shfl_xor(hm, 32, 64));
        if (hm > m[pp]) {
          l[pp] = m[pp] == -INFINITY ? 0.f : l[pp] * exp2f(m[pp] - hm);
          m[pp] = hm;
        }
        if (m[pp] != -INFINITY) {
#pragma unroll
          for (int ii = 0; ii < 4; ++ii) l[pp] += exp2f(v[ii] - m[pp]);
        }
      }
    }
    if (loader && t + 1 < ntiles) *reinterpret_cast<u32x4*>(&kt[buf ^ 1][lk][8 * lc]) = nxt;
    __syncthreads();
  }
#pragma unroll
  for (int pp = 0; pp < HP_PPW; ++pp) {
    float lt = l[pp];
    lt += __shfl_xor(lt, 16, 64);
    lt += __shfl_xor(lt, 32, 64);
    const int pos = p_w + pp;
    if (g == 0 && c16 < a.G && pos < L) a.lse2[(size_t(unit) * a.G + c16) * L + pos] = m[pp] + log2f(lt);
  }
}

template <int D>
__global__ __launch_bounds__(512) void hp_colsum_kernel(HpArgs a) {
  constexpr int NKS = D / 32, PITCH = D + 8, CH = D / 8;
  constexpr int TCH = HP_QT * 16 * CH;                  // 16-byte chunks of one Q tile (16 head rows per position)
  constexpr int TPT = (TCH + 511) / 512;                // chunks per thread
  __shared__ __align__(16) uint16_t qt[2][HP_QT][16][PITCH];
  __shared__ float lt[2][HP_QT][16];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, g = lane >> 4, c16 = lane & 15;
  const int unit = blockIdx.y, b = unit / a.Hkv, kvh = unit % a.Hkv;
  const int L = a.L, j_blk = blockIdx.x * HP_KEYS;
  if (j_blk >= L) return;                               // uniform per block
  const uint16_t* ku = a.k + size_t(unit) * a.cap * D;
  const uint16_t* qu = a.q + (size_t(b) * a.Hq + size_t(kvh) * a.G) * size_t(L) * D;
  const float* lu = a.lse2 + size_t(unit) * a.G * L;
  // this wave's keys: j_w + 16 kb + c16 as A rows
  const int j_w = j_blk + w * HP_KB * 16;
  u32x4 ak[HP_KB][NKS];
#pragma unroll
  for (int kb = 0; kb < HP_KB; ++kb) {
    const int key = min(j_w + 16 * kb + c16, L - 1);
#pragma unroll
    for (int c = 0; c < NKS; ++c) ak[kb][c] = ld16(ku + size_t(key) * D + 8 * g + 32 * c);
  }
  float col[HP_KB][4];
#pragma unroll
  for (int kb = 0; kb < HP_KB; ++kb)
#pragma unroll
    for (int ii = 0; ii < 4; ++ii) col[kb][ii] = 0.f;
  const int i_end = L, i_beg = j_blk;                   // queries before the block's first key give it nothing
  const int ntiles = (i_end - i_beg + HP_QT - 1) / HP_QT;
  // Q tile chunk e: position e / (16 CH), head (e / CH) % 16, chunk e % CH (zeros for heads >= G or past L)
  u32x4 stage[TPT];
  float lstage = 0.f;
  auto fetch = [&](int t) {
#pragma unroll
    for (int j = 0; j < TPT; ++j) {
      const int e = threadIdx.x + 512 * j;
      const int pp = e / (16 * CH), h = (e / CH) % 16, ch = e % CH;
      const int pos = i_beg + t * HP_QT + pp;
      const bool ok = e < TCH && h < a.G && pos < L;
      stage[j] = ok ? ld16(qu + (size_t(h) * L + pos) * D + 8 * ch) : u32x4{0, 0, 0, 0};
    }
    if (threadIdx.x < HP_QT * 16) {
      const int pp = threadIdx.x / 16, h = threadIdx.x % 16, pos = i_beg + t * HP_QT + pp;
      lstage = (h < a.G && pos < L) ? lu[size_t(h) * L + pos] : 0.f;
    }
  };
  auto put = [&](int buf) {
#pragma unroll
    for (int j = 0; j < TPT; ++j) {
      const int e = threadIdx.x + 512 * j;
      if (e < TCH) *reinterpret_cast<u32x4*>(&qt[buf][e / (16 * CH)][(e / CH) % 16][8 * (e % CH)]) = stage[j];
    }
    if (threadIdx.x < HP_QT * 16) lt[buf][threadIdx.x / 16][threadIdx.x % 16] = lstage;
  };
  fetch(0);
  put(0);
  __syncthreads();
  for (int t = 0; t < ntiles; ++t) {
    const int buf = t & 1;
    if (t + 1 < ntiles) fetch(t + 1);
#pragma unroll
    for (int pp = 0; pp < HP_QT; ++pp) {
      const int pos = i_beg + t * HP_QT + pp;
      if (pos >= L) break;                              // uniform across the block
      u32x4 bq[NKS];
#pragma unroll
      for (int c = 0; c < NKS; ++c) bq[c] = *reinterpret_cast<const u32x4*>(&qt[buf][pp][c16][8 * g + 32 * c]);
      const float lse = lt[buf][pp][c16];
      const bool head_ok = c16 < a.G;
#pragma unroll
      for (int kb = 0; kb < HP_KB; ++kb) {
        if (j_w + 16 * kb > pos) continue;              // every key of this block comes after the query
        f32x4 s = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int c = 0; c < NKS; ++c) s = mfma_bf16_16x16x32(ak[kb][c], bq[c], s);
#pragma unroll
        for (int ii = 0; ii < 4; ++ii) {
          const int key = j_w + 16 * kb + 4 * g + ii;
          if (head_ok && key <= pos) col[kb][ii] += exp2f(s[ii] * a.sc2 - lse);
        }
      }
    }
    if (t + 1 < ntiles) put(buf ^ 1);
    __syncthreads();
  }
  // sum over the 16 head lanes of each key
#pragma unroll
  for (int kb = 0; kb < HP_KB; ++kb)
#pragma unroll
    for (int ii = 0; ii < 4; ++ii) {
      float v = col[kb][ii];
#pragma unroll
      for (int o = 1; o < 16; o <<= 1) v += __shfl_xor(v, o, 64);
      const int key = j_w + 16 * kb + 4 * g + ii;
      if (c16 == 0 && key < L) {
        a.acc0[size_t(unit) * L + key] = v;
        if (key < a.n_cand) a.votes[size_t(unit) * a.n_cand + key] = v;
      }
    }
}

// Slot state from the kept positions: slot_pos[i] = kept[i], acc[i] = acc0[kept[i]]
// for i < n, -1 / 0 for the remaining slots.
__global__ __launch_bounds__(256) void hp_state_kernel(const int32_t* __restrict__ kept, int kept_stride,
                                                       const int32_t* __restrict__ kept_len,
                                                       const float* __restrict__ acc0, int L, int32_t* __restrict__ slot_pos,
                                                       float* __restrict__ acc, int cap, int Hkv) {
  const int unit = blockIdx.x, b = unit / Hkv;
  const int n = min(kept_len[b], min(kept_stride, cap));
  for (int i = threadIdx.x; i < cap; i += blockDim.x) {
    const int p = i < n ? kept[size_t(unit) * kept_stride + i] : -1;
    const bool ok = p >= 0 && p < L;
    slot_pos[size_t(unit) * cap + i] = ok ? p : -1;
    acc[size_t(unit) * cap + i] = ok ? acc0[size_t(unit) * L + p] : 0.f;
  }
}

se_status launch_h2o_prefill_scores(const se_cache& c, const void* q, const void* k, int L, int n_cand, float scale,
                                    float* lse2, float* acc0, float* votes, hipStream_t s) {
  HpArgs a{};
  a.q = (const uint16_t*)q; a.k = (const uint16_t*)k; a.lse2 = lse2; a.acc0 = acc0; a.votes = votes;
  a.Hq = c.n_q_heads; a.Hkv = c.n_kv_heads; a.G = c.n_q_heads / c.n_kv_heads; a.cap = c.capacity; a.L = L;
  a.n_cand = n_cand;
  a.sc2 = scale * 1.4426950408889634f;
  const int units = c.batch * c.n_kv_heads;
  const dim3 ga(ceil_div(L, HP_POS), units), gb(ceil_div(L, HP_KEYS), units);
  if (c.d_k == 128) {
    hipLaunchKernelGGL(hp_rowlse_kernel<128>, ga, dim3(512), 0, s, a);
    hipLaunchKernelGGL(hp_colsum_kernel<128>, gb, dim3(512), 0, s, a);
  } else {
    hipLaunchKernelGGL(hp_rowlse_kernel<64>, ga, dim3(512), 0, s, a);
    hipLaunchKernelGGL(hp_colsum_kernel<64>, gb, dim3(512), 0, s, a);
  }
  return launch_status();
}

se_status launch_h2o_state(const se_cache& c_slots, const int32_t* kept, int kept_stride, const int32_t* kept_len,
                           const float* acc0, int L, int32_t* slot_pos, float* acc, hipStream_t s) {
  hipLaunchKernelGGL(hp_state_kernel, dim3(c_slots.batch * c_slots.n_kv_heads), dim3(256), 0, s, kept, kept_stride,
                     kept_len, acc0, L, slot_pos, acc, c_slots.capacity, c_slots.n_kv_heads);
  return launch_status();
}

}  // namespace se
