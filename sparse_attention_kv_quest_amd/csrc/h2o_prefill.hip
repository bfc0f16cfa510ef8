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
// Both compute S^T[key][row] = K . Q^T on 16x16x32 MFMA: A = 16 keys (lane: key
// c16, dims 32c + 8g ..), B = 16 consecutive (position, head) query rows (lane:
// row c16, the same dims).  K tiles (pass A, 12-wave blocks at three waves per
// SIMD) and Q tiles (pass B, 8-wave blocks) go through double-buffered LDS shared
// by the block's waves.  Both passes are bound by the vector ALU (one exp2 and two
// to five other operations per score), so the MFMAs of the next 16x16 score tile
// are issued before the exps of the current one.
// The kept set then follows the SnapKV keep rule on acc0 (no pooling).
#include "se_internal.hpp"
#include "mfma_util.hpp"

namespace se {

constexpr int HPA_WAVES = 12;                   // pass A: waves per block
constexpr int HPA_THREADS = 64 * HPA_WAVES;
constexpr int HP_NG = 4;                        // pass A: 16-row groups per wave
constexpr int HP_RPW = HP_NG * 16;              // pass A: (position, head) rows per wave
constexpr int HP_ROWS = HPA_WAVES * HP_RPW;     // pass A: 768 rows per block
constexpr int HP_KT = 64;                       // pass A: keys per K tile
constexpr int HPB_WAVES = 8;                    // pass B: waves per block
constexpr int HPB_THREADS = 64 * HPB_WAVES;
constexpr int HP_KB = 4;                        // pass B: 16-key blocks per wave
constexpr int HP_KEYS = HPB_WAVES * HP_KB * 16; // pass B: 512 keys per block
constexpr int HP_QR = 128;                      // pass B: (position, head) rows per Q tile
constexpr float HP_MARGIN = 8.f;                // pass A: log2 headroom before the running max moves

struct HpArgs {
  const uint16_t* q;    // [B][Hq][L][D] every prompt query
  const uint16_t* k;    // [B][Hkv][cap][D]
  float* lse2;          // [units][L * G], row r = position r / G, head r % G
  float* acc0;          // [units][L]
  float* votes;         // [units][L - recent]: acc0 of the candidates of the keep rule
  int Hq, Hkv, G, cap, L, n_cand;
  int units;            // batch * Hkv
  float sc2;            // scale * log2(e)
};

// Eight floats as separate fields, indexed only by unrolled constants.  An array
// indexed that way becomes one 8-wide vector value after unrolling, and the
// compiler then copies the whole register tuple at every branch join.
struct F8 {
  float v0, v1, v2, v3, v4, v5, v6, v7;
  __device__ __forceinline__ float& operator[](int i) {
    switch (i) {
      case 0: return v0; case 1: return v1; case 2: return v2; case 3: return v3;
      case 4: return v4; case 5: return v5; case 6: return v6; default: return v7;
    }
  }
};

// The group's queries are taken as L * G rows (position-major, head-minor) and go
// sixteen at a time into the MFMA N dimension, so no column is spent on padding
// whatever G is.

template <int D>
__global__ __launch_bounds__(HPA_THREADS) void hp_rowlse_kernel(HpArgs a) {
  constexpr int NKS = D / 32, PITCH = D + 8, CH = D / 8;   // CH 16-byte chunks per row
  constexpr int NCH = HP_KT * CH, TPT = (NCH + HPA_THREADS - 1) / HPA_THREADS;   // K tile chunks (per thread)
  __shared__ __align__(16) uint16_t kt[2][HP_KT][PITCH];
  const int lane = threadIdx.x & 63, g = lane >> 4, c16 = lane & 15;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int unit = blockIdx.x % a.units, b = unit / a.Hkv, kvh = unit % a.Hkv;
  const int L = a.L, G = a.G, nrows = L * G;
  const int r_blk = ((nrows + HP_ROWS - 1) / HP_ROWS - 1 - int(blockIdx.x / a.units)) * HP_ROWS;   // latest rows first
  if (r_blk >= nrows) return;                          // uniform per block
  const int r_w = r_blk + w * HP_RPW;
  const uint16_t* ku = a.k + size_t(unit) * a.cap * D;
  const uint16_t* qu = a.q + (size_t(b) * a.Hq + size_t(kvh) * G) * size_t(L) * D;
  u32x4 qv[HP_NG][NKS];
  int lpos[HP_NG], pmin[HP_NG], pmax[HP_NG];
#pragma unroll
  for (int j = 0; j < HP_NG; ++j) {
    const int r = r_w + 16 * j + c16;
    const bool ok = r < nrows;
    lpos[j] = r / G;
    pmin[j] = (r_w + 16 * j) / G;                      // wave-uniform bounds of the group's positions
    pmax[j] = (r_w + 16 * j + 15) / G;
    const uint16_t* qp = qu + (ok ? (size_t(r % G) * L + r / G) * D : 0);
#pragma unroll
    for (int c = 0; c < NKS; ++c) qv[j][c] = ok ? ld16(qp + 8 * g + 32 * c) : u32x4{0, 0, 0, 0};
  }
  static_assert(HP_NG <= 8, "one F8 field per row group");
  F8 m, l;
#pragma unroll
  for (int j = 0; j < HP_NG; ++j) { m[j] = -INFINITY; l[j] = 0.f; }
  const int last_pos = (min(nrows, r_blk + HP_ROWS) - 1) / G;
  const int ntiles = last_pos / HP_KT + 1;             // keys up to the block's last position
  u32x4 stage[TPT];
  auto fetch = [&](int t) {
#pragma unroll
    for (int i = 0; i < TPT; ++i) {
      const int e = threadIdx.x + HPA_THREADS * i;
      const int key = min(t * HP_KT + e / CH, L - 1);
      if (NCH % HPA_THREADS == 0 || e < NCH) stage[i] = ld16(ku + size_t(key) * D + 8 * (e % CH));
    }
  };
  auto put = [&](int buf) {
#pragma unroll
    for (int i = 0; i < TPT; ++i) {
      const int e = threadIdx.x + HPA_THREADS * i;
      if (NCH % HPA_THREADS == 0 || e < NCH) *reinterpret_cast<u32x4*>(&kt[buf][e / CH][8 * (e % CH)]) = stage[i];
    }
  };
  fetch(0);
  put(0);
  __syncthreads();
  for (int t = 0; t < ntiles; ++t) {
    const int buf = t & 1;
    if (t + 1 < ntiles) fetch(t + 1);
    if (t * HP_KT + HP_KT - 1 <= pmin[0]) {            // every key of the tile precedes every row of the wave
      // software pipeline over the tile's (16-key block, row group) pairs: the next
      // pair's scores go through the matrix cores while this pair's max test and exps
      // run; the next key block's operands are read from LDS a block ahead
      constexpr int NSB = HP_KT / 16, NP = NSB * HP_NG;
      u32x4 ak[2][NKS];
      auto rd = [&](int sb) {
#pragma unroll
        for (int c = 0; c < NKS; ++c)
          ak[sb & 1][c] = *reinterpret_cast<const u32x4*>(&kt[buf][16 * sb + c16][8 * g + 32 * c]);
      };
      auto mm = [&](int p) {
        const int sb = p / HP_NG, j = p % HP_NG;
        f32x4 r = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int c = 0; c < NKS; ++c) r = mfma_bf16_16x16x32(ak[sb & 1][c], qv[j][c], r);
        return r;
      };
      // raw score above which a key moves the running max: (m + margin) / sc2
      const float inv_sc2 = 1.f / a.sc2;
      F8 thr;
#pragma unroll
      for (int j = 0; j < HP_NG; ++j) thr[j] = (m[j] + HP_MARGIN) * inv_sc2;
      rd(0);
      f32x4 sc = mm(0);
#pragma unroll
      for (int p = 0; p < NP; ++p) {
        const int sb = p / HP_NG, j = p % HP_NG;
        if (j == 0 && sb + 1 < NSB) rd(sb + 1);
        f32x4 sn = sc;
        if (p + 1 < NP) sn = mm(p + 1);
        // the running max moves only when a key beats it by more than 2^8, which is
        // rare once a row has seen a few keys: the raw scores are compared with that
        // bound in raw units, and one wave-uniform test per pair takes the update
        const bool up = (sc[0] > thr[j]) | (sc[1] > thr[j]) | (sc[2] > thr[j]) | (sc[3] > thr[j]);
        if (__builtin_amdgcn_ballot_w64(up)) {
          const float hm = fmaxf(fmaxf(sc[0], sc[1]), fmaxf(sc[2], sc[3])) * a.sc2;
          l[j] = up ? (m[j] == -INFINITY ? 0.f : l[j] * ex2(m[j] - hm)) : l[j];
          thr[j] = up ? (hm + HP_MARGIN) * inv_sc2 : thr[j];
          m[j] = up ? hm : m[j];
        }
#pragma unroll
        for (int ii = 0; ii < 4; ++ii) l[j] += ex2(fmaf(sc[ii], a.sc2, -m[j]));
        // keeps the sum here: left free, the compiler sinks it to the row group's next
        // pair and holds the scores of the pairs between in registers
        asm volatile("" : "+v"(l[j]));
        sc = sn;
      }
      if (t + 1 < ntiles) put(buf ^ 1);
      __syncthreads();
      continue;
    }
#pragma unroll
    for (int sb = 0; sb < HP_KT / 16; ++sb) {
      const int key0 = t * HP_KT + 16 * sb;
      if (key0 > pmax[HP_NG - 1]) break;               // later than every position of the wave
      u32x4 ak[NKS];
#pragma unroll
      for (int c = 0; c < NKS; ++c) ak[c] = *reinterpret_cast<const u32x4*>(&kt[buf][16 * sb + c16][8 * g + 32 * c]);
      const int kbase = key0 + 4 * g;
#pragma unroll
      for (int j = 0; j < HP_NG; ++j) {
        if (key0 > pmax[j]) continue;                  // every key of the block comes later
        f32x4 s = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int c = 0; c < NKS; ++c) s = mfma_bf16_16x16x32(ak[c], qv[j][c], s);
        float v[4];
        if (key0 + 15 <= pmin[j]) {                    // the whole block is causal for the group
#pragma unroll
          for (int ii = 0; ii < 4; ++ii) v[ii] = s[ii] * a.sc2;
        } else {
#pragma unroll
          for (int ii = 0; ii < 4; ++ii) v[ii] = kbase + ii <= lpos[j] ? s[ii] * a.sc2 : -INFINITY;
        }
        // this lane's own keys: running max moved only when exceeded by more than 2^8
        const float hm = fmaxf(fmaxf(v[0], v[1]), fmaxf(v[2], v[3]));
        if (hm > m[j] + HP_MARGIN) {
          l[j] = m[j] == -INFINITY ? 0.f : l[j] * ex2(m[j] - hm);
          m[j] = hm;
        }
        const float mr = m[j] == -INFINITY ? 0.f : m[j];
#pragma unroll
        for (int ii = 0; ii < 4; ++ii) l[j] += ex2(v[ii] - mr);
      }
    }
    if (t + 1 < ntiles) put(buf ^ 1);
    __syncthreads();
  }
  // merge the four lanes of each row: they saw disjoint keys; lanes that saw none
  // (m = -inf) add nothing, and key 0 makes the row's maximum finite
#pragma unroll
  for (int j = 0; j < HP_NG; ++j) {
    const float mt = rows4_max(m[j]);
    float lt = m[j] == -INFINITY ? 0.f : l[j] * ex2(m[j] - mt);
    lt = rows4_sum(lt);
    const int r = r_w + 16 * j + c16;
    if (g == 0 && r < nrows) a.lse2[size_t(unit) * nrows + r] = mt + log2f(lt);
  }
}

template <int D>
__global__ __launch_bounds__(HPB_THREADS) void hp_colsum_kernel(HpArgs a) {
  constexpr int NKS = D / 32, PITCH = D + 8, CH = D / 8;
  constexpr int TPT = HP_QR * CH / HPB_THREADS;         // Q tile chunks per thread
  constexpr int NQG = HP_QR / 16;                       // 16-row groups per Q tile
  __shared__ __align__(16) uint16_t qt[2][HP_QR][PITCH];
  __shared__ float lt[2][HP_QR];
  const int lane = threadIdx.x & 63, g = lane >> 4, c16 = lane & 15;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int unit = blockIdx.x % a.units, b = unit / a.Hkv, kvh = unit % a.Hkv;
  const int L = a.L, G = a.G, nrows = L * G;
  const int j_blk = int(blockIdx.x / a.units) * HP_KEYS;   // the earliest keys (most rows) first
  if (j_blk >= L) return;                               // uniform per block
  const uint16_t* ku = a.k + size_t(unit) * a.cap * D;
  const uint16_t* qu = a.q + (size_t(b) * a.Hq + size_t(kvh) * G) * size_t(L) * D;
  const float* lu = a.lse2 + size_t(unit) * nrows;
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
  const int r_beg = j_blk * G;                          // rows of earlier positions give the block nothing
  const int r_full = (j_blk + HP_KEYS) * G;             // rows from here on come after every key of the block
  const int ntiles = (nrows - r_beg + HP_QR - 1) / HP_QR;
  // Q tile chunk e: row e / CH, chunk e % CH; rows past the end are zero with lse +inf (weight 0)
  u32x4 stage[TPT];
  float lstage = 0.f;
  auto fetch = [&](int t) {
    const int r0 = r_beg + t * HP_QR;
#pragma unroll
    for (int i = 0; i < TPT; ++i) {
      const int e = threadIdx.x + HPB_THREADS * i;
      const int r = r0 + e / CH;
      stage[i] = r < nrows ? ld16(qu + (size_t(r % G) * L + r / G) * D + 8 * (e % CH)) : u32x4{0, 0, 0, 0};
    }
    if (threadIdx.x < HP_QR) lstage = r0 + int(threadIdx.x) < nrows ? lu[r0 + threadIdx.x] : INFINITY;
  };
  auto put = [&](int buf) {
#pragma unroll
    for (int i = 0; i < TPT; ++i) {
      const int e = threadIdx.x + HPB_THREADS * i;
      *reinterpret_cast<u32x4*>(&qt[buf][e / CH][8 * (e % CH)]) = stage[i];
    }
    if (threadIdx.x < HP_QR) lt[buf][threadIdx.x] = lstage;
  };
  fetch(0);
  put(0);
  __syncthreads();
  for (int t = 0; t < ntiles; ++t) {
    const int buf = t & 1, r0 = r_beg + t * HP_QR;
    if (t + 1 < ntiles) fetch(t + 1);
    if (r0 >= r_full && r0 + HP_QR <= nrows) {         // a whole tile, no causal test anywhere
      // software pipeline over the tile's 16-row groups: the scores of group j + 1 go
      // through the matrix cores while group j's exps run, and group j + 2's operands
      // are read from LDS meanwhile
      u32x4 bq[NQG][NKS];
      float nl[NQG];
      f32x4 s[NQG][HP_KB];
      auto rd = [&](int j) {
#pragma unroll
        for (int c = 0; c < NKS; ++c) bq[j][c] = *reinterpret_cast<const u32x4*>(&qt[buf][16 * j + c16][8 * g + 32 * c]);
        nl[j] = -lt[buf][16 * j + c16];
      };
      auto mm = [&](int j) {
#pragma unroll
        for (int kb = 0; kb < HP_KB; ++kb) s[j][kb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int c = 0; c < NKS; ++c)
#pragma unroll
          for (int kb = 0; kb < HP_KB; ++kb) s[j][kb] = mfma_bf16_16x16x32(ak[kb][c], bq[j][c], s[j][kb]);
      };
      rd(0);
      rd(1);
      mm(0);
#pragma unroll
      for (int j = 0; j < NQG; ++j) {
        if (j + 2 < NQG) rd(j + 2);
        if (j + 1 < NQG) mm(j + 1);
#pragma unroll
        for (int kb = 0; kb < HP_KB; ++kb)
#pragma unroll
          for (int ii = 0; ii < 4; ++ii) col[kb][ii] += ex2(fmaf(s[j][kb][ii], a.sc2, nl[j]));
        if (j + 1 < NQG) {
          if (j + 2 < NQG) __builtin_amdgcn_sched_group_barrier(0x100, NKS + 1, 0);
#pragma unroll
          for (int i = 0; i < NKS * HP_KB; ++i) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x002, 3, 0);
          }
        }
        __builtin_amdgcn_sched_barrier(0);             // one scheduling region per group
      }
    } else if (r0 >= r_full) {                          // the partial last tile
#pragma unroll
      for (int j = 0; j < NQG; ++j) {
        if (r0 + 16 * j >= nrows) break;                // uniform across the block
        u32x4 bq[NKS];
#pragma unroll
        for (int c = 0; c < NKS; ++c) bq[c] = *reinterpret_cast<const u32x4*>(&qt[buf][16 * j + c16][8 * g + 32 * c]);
        const float nlse = -lt[buf][16 * j + c16];
#pragma unroll
        for (int kb = 0; kb < HP_KB; ++kb) {
          f32x4 s = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int c = 0; c < NKS; ++c) s = mfma_bf16_16x16x32(ak[kb][c], bq[c], s);
#pragma unroll
          for (int ii = 0; ii < 4; ++ii) col[kb][ii] += ex2(fmaf(s[ii], a.sc2, nlse));
        }
      }
    } else {
#pragma unroll
      for (int j = 0; j < NQG; ++j) {
        const int rg = r0 + 16 * j;
        if (rg >= nrows) break;                         // uniform across the block
        const int pmin = rg / G, pmax = (rg + 15) / G, lpos = (rg + c16) / G;
        u32x4 bq[NKS];
#pragma unroll
        for (int c = 0; c < NKS; ++c) bq[c] = *reinterpret_cast<const u32x4*>(&qt[buf][16 * j + c16][8 * g + 32 * c]);
        const float nlse = -lt[buf][16 * j + c16];
#pragma unroll
        for (int kb = 0; kb < HP_KB; ++kb) {
          if (j_w + 16 * kb > pmax) continue;           // every key of this block comes after the group
          f32x4 s = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int c = 0; c < NKS; ++c) s = mfma_bf16_16x16x32(ak[kb][c], bq[c], s);
          if (j_w + 16 * kb + 15 <= pmin) {
#pragma unroll
            for (int ii = 0; ii < 4; ++ii) col[kb][ii] += ex2(fmaf(s[ii], a.sc2, nlse));
          } else {
#pragma unroll
            for (int ii = 0; ii < 4; ++ii) {
              const int key = j_w + 16 * kb + 4 * g + ii;
              if (key <= lpos) col[kb][ii] += ex2(fmaf(s[ii], a.sc2, nlse));
            }
          }
        }
      }
    }
    if (t + 1 < ntiles) put(buf ^ 1);
    __syncthreads();
  }
  // sum over the 16 row lanes of each key
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
  // Block b takes unit b % units: a block fills a CU, and the dispatcher then deals
  // consecutive blocks to the CUs in a fixed rotation, so consecutive blocks should cost
  // the same (one causal row / key block of every unit) and each CU should see every
  // block index.  With the units outermost, each CU had received the same block index
  // of every unit, from the cheapest to the costliest, and the launch ran twice as long
  // as the average CU's work.
  a.units = units;
  if (int64_t(units) * std::max(ceil_div(L * a.G, HP_ROWS), ceil_div(L, HP_KEYS)) > INT32_MAX) return SE_ERR_SHAPE;
  const dim3 ga(units * ceil_div(L * a.G, HP_ROWS)), gb(units * ceil_div(L, HP_KEYS));
  if (c.d_k == 128) {
    hipLaunchKernelGGL(hp_rowlse_kernel<128>, ga, dim3(HPA_THREADS), 0, s, a);
    hipLaunchKernelGGL(hp_colsum_kernel<128>, gb, dim3(HPB_THREADS), 0, s, a);
  } else {
    hipLaunchKernelGGL(hp_rowlse_kernel<64>, ga, dim3(HPA_THREADS), 0, s, a);
    hipLaunchKernelGGL(hp_colsum_kernel<64>, gb, dim3(HPB_THREADS), 0, s, a);
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
