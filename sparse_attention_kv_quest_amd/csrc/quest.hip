// Quest page scoring and top-k page view.
//
// tokendh.com explainer, section "历史太长,会撑爆什么": Quest chooses pages per
// query from a summary index kept beside the full history.  A page's score for
// query head h is the upper bound sum_d max(q_hd * min_pd, q_hd * max_pd) of
// q_h . k over the page, i.e. sum_d (q+_hd * max_pd + q-_hd * min_pd) with
// q+ = max(q, 0), q- = min(q, 0); a KV head's page score is the max over the
// heads of its group.  The view is the top pages (ties to the lower page),
// in ascending page order.
//
// bf16 caches score on MFMA: the bound of every (page, head) pair is one dense
// contraction S^T = [max | min] . [q+ | q-]^T over 2 d_k terms, whose partial
// sums are exact in fp32 for the grid-valued inputs the tests use.  fp32 caches
// use the vector kernel.
#include "fp8_row.hpp"
#include "mfma_util.hpp"

namespace se {

constexpr int QUEST_TOPK_LDS = 8192;  // page scores held in LDS by the block top-k kernel

// ------------------------------------------------------------------ vector scoring (fp32 / fallback)
// grid: (page blocks, units); block 256 threads = PPB pages x G heads (G <= 64).
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

// ------------------------------------------------------------------ MFMA scoring (bf16)
// grid: (page groups, units); 4 waves, each scoring one block of 16 pages, with
// every metadata load issued before q is staged in LDS.
// A operand of k-step s: lane (g, c) reads dims 32s + 8g .. 32s + 8g + 7 of page c's max (then min) row;
// B operand: q+ (then q-) of head c (+16 per head block), the same dims, staged in
// LDS in lane order.  Result lane (g, c): pages 4g..4g+3, head c.
//
// APP (the fused decode call): before scoring, the new token's K / V rows are
// written at slot seq_len[b] and the new row is folded into the min / max of the
// page receiving it (kmin / kmax hold each page's in-order min / max, as every
// call here leaves them, so this equals the separate call's rebuild bit for
// bit).  Pages are counted with the new length; seq_len itself is left for the
// top-k launch to update, after every block of the batch row has read it.
//
// APP == 2 (the fused FP8 decode step): the new rows are stored as FP8 codes and
// scale bytes (the encoding of fp8_row.hpp, as se_kv_append_fp8 writes them), and the
// stored values of the new K row are folded into the page's min / max.
struct QuestAppendArgs {
  uint16_t* k; uint16_t* v;                      // cache rows [units][cap][D]; v null for a latent cache
  const uint16_t* k_new; const uint16_t* v_new;  // [units][D]
  uint16_t* kmin_w; uint16_t* kmax_w;            // the metadata, written for the appended page
  uint8_t* kq; uint8_t* vq; uint8_t* ks; uint8_t* vs;   // APP == 2: codes [units][cap][D], scales [units][cap]
};

__device__ __forceinline__ uint32_t bf16x2_fmin(uint32_t acc, uint32_t x, bool mx) {
  const float lo = mx ? fmaxf(bf16_lo(acc), bf16_lo(x)) : fminf(bf16_lo(acc), bf16_lo(x));
  const float hi = mx ? fmaxf(bf16_hi(acc), bf16_hi(x)) : fminf(bf16_hi(acc), bf16_hi(x));
  return (__float_as_uint(lo) >> 16) | (__float_as_uint(hi) & 0xffff0000u);
}

// Eight blocks per CU for one head block: a Quest 32K grid (2112 blocks) then takes
// one round of the GPU but for 64 blocks, where seven per CU left 320 for a second.
template <int D, int HB, int APP>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(HB == 1 ? 8 : 1, 8))) void quest_score_mfma_kernel(
    const uint16_t* __restrict__ q, const uint16_t* kmin, const uint16_t* kmax,
    const int32_t* seq_len, float* score, int Hkv, int G, int P, int ncp, int cap, QuestAppendArgs ap) {
  constexpr int NKS = D / 32;
  __shared__ u32x4 qb[2 * NKS][HB][64];
  __shared__ __align__(16) uint16_t frow[APP == 2 ? D : 8];   // FP8 append: the new K row as stored (bf16)
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, g = lane >> 4, c16 = lane & 15;
  const int unit = blockIdx.y, b = unit / Hkv, kvh = unit % Hkv;
  const int len = min(seq_len[b], cap);
  const bool app = APP && len < cap;                 // room for the new token
  const int new_len = app ? len + 1 : len;
  const int npages = min((new_len + P - 1) / P, ncp);
  // q first (each 16-byte piece feeds both the q+ and the q- entry), then the
  // page metadata: all in flight together, and q's wait leaves the metadata
  // loads outstanding.  Unconditional loads (a clamped entry and head; pages past
  // the last valid one read page 0, their scores masked below) keep the wait
  // counters exact.
  const uint16_t* qg = q + (size_t(b) * Hkv * G + size_t(kvh) * G) * D;
  constexpr int QE = NKS * HB * 64, QR = (QE + 255) / 256;
  u32x4 qv[QR];
#pragma unroll
  for (int t = 0; t < QR; ++t) {
    const int idx = min(int(threadIdx.x) + 256 * t, QE - 1);
    const int ln = idx & 63, hb = (idx >> 6) % HB, c = idx / (64 * HB);
    const int head = 16 * hb + (ln & 15);
    qv[t] = ld16(qg + size_t(min(head, G - 1)) * D + 32 * c + 8 * (ln >> 4));
  }
  __builtin_amdgcn_sched_barrier(0);   // q's loads stay ahead of the metadata's
  u32x4 amx[NKS], amn[NKS];
  const int pg = (blockIdx.x * 4 + w) * 16 + c16;
  {
    const bool ok = pg < npages;
    const uint16_t* mxp = kmax + (size_t(unit) * ncp + (ok ? pg : 0)) * D + 8 * g;
    const uint16_t* mnp = kmin + (size_t(unit) * ncp + (ok ? pg : 0)) * D + 8 * g;
#pragma unroll
    for (int c = 0; c < NKS; ++c) {
      amx[c] = ld16(mxp + 32 * c);
      amn[c] = ld16(mnp + 32 * c);
    }
  }
  // folds a new K row (bf16 values, this lane's dims 8g + 32c) into the min / max of
  // page plast: the page's stored values with the new row folded in (the last step of
  // the in-order rebuild the separate calls run, so bit-identical), or the new row
  // alone on a fresh page; the page is then scored from the folded rows
  auto fold_new_row = [&](const u32x4 (&xk)[NKS], int plast) {
    const bool fresh = len % P == 0;
    const size_t mo = (size_t(unit) * ncp + plast) * D + 8 * g;
#pragma unroll
    for (int c = 0; c < NKS; ++c) {
      const u32x4 x = xk[c];
      u32x4 mn, mx;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        mn[j] = bf16x2_fmin(fresh ? 0x7f807f80u : amn[c][j], x[j], false);   // +inf pair on a fresh page
        mx[j] = bf16x2_fmin(fresh ? 0xff80ff80u : amx[c][j], x[j], true);    // -inf pair
      }
      *reinterpret_cast<u32x4*>(ap.kmin_w + mo + 32 * c) = mn;
      *reinterpret_cast<u32x4*>(ap.kmax_w + mo + 32 * c) = mx;
      amn[c] = mn;
      amx[c] = mx;
    }
  };
  if (APP && app) {
    const int plast = len / P;
    const size_t urow = size_t(unit) * cap;
    if (blockIdx.x == plast / 64) {   // this block writes the new K / V rows
      if constexpr (APP == 2) {
        constexpr int TPR = D / 8;        // threads per row: K's first, then V's
        if (threadIdx.x < 2 * TPR) {
          const bool isv = threadIdx.x >= TPR;
          const int part = threadIdx.x % TPR;
          int e;
          const uint2 cw = fp8_quantize8<TPR>(ld16((isv ? ap.v_new : ap.k_new) + size_t(unit) * D + 8 * part), e);
          *reinterpret_cast<uint2*>((isv ? ap.vq : ap.kq) + (urow + len) * D + 8 * part) = cw;
          if (part == 0) (isv ? ap.vs : ap.ks)[urow + len] = uint8_t(e + 127);
          if (!isv) {   // the stored K values (exact in bf16) for the page's min / max below
            u32x4 sv;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
              const uint32_t wd = j < 2 ? cw.x : cw.y;
              const float lo = (j & 1) ? fp8_value<2>(wd, e) : fp8_value<0>(wd, e);
              const float hi = (j & 1) ? fp8_value<3>(wd, e) : fp8_value<1>(wd, e);
              sv[j] = (__float_as_uint(lo) >> 16) | (__float_as_uint(hi) & 0xffff0000u);
            }
            *reinterpret_cast<u32x4*>(&frow[8 * part]) = sv;
          }
        }
      } else {
        for (int i = threadIdx.x; i < 2 * (D / 8); i += 256) {
          const bool isv = i >= D / 8;
          const int o = 8 * (isv ? i - D / 8 : i);
          if (!isv) *reinterpret_cast<u32x4*>(ap.k + (urow + len) * D + o) = ld16(ap.k_new + size_t(unit) * D + o);
          else if (ap.v != nullptr)
            *reinterpret_cast<u32x4*>(ap.v + (urow + len) * D + o) = ld16(ap.v_new + size_t(unit) * D + o);
        }
      }
    }
    if (APP == 1 && pg == plast) {   // this lane's dims of the new row, folded into the page
      const uint16_t* kn = ap.k_new + size_t(unit) * D + 8 * g;
      u32x4 xk[NKS];   // all of the new row's pieces in flight before the stores
#pragma unroll
      for (int c = 0; c < NKS; ++c) xk[c] = ld16(kn + 32 * c);
      fold_new_row(xk, plast);
    }
  }
  // threads past the last entry store that entry again (the same values): no branch
  // for the compiler to sink a load into
#pragma unroll
  for (int t = 0; t < QR; ++t) {
    const int idx = min(int(threadIdx.x) + 256 * t, QE - 1);
    const int ln = idx & 63, hb = (idx >> 6) % HB, c = idx / (64 * HB);
    const int head = 16 * hb + (ln & 15);
    const u32x4 x = head < G ? qv[t] : u32x4{0, 0, 0, 0};
    u32x4 xp, xn;
    // q- keeps the halves whose sign bit is set, q+ the others
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint32_t sgn = ((x[j] >> 15) & 1u) * 0xffffu | ((x[j] >> 31) & 1u) * 0xffff0000u;
      xp[j] = x[j] & ~sgn;
      xn[j] = x[j] & sgn;
    }
    qb[c][hb][ln] = xp;
    qb[NKS + c][hb][ln] = xn;
  }
  __syncthreads();
  if constexpr (APP == 2) {
    // FP8 append: the new K row as stored (written to LDS by the block's row writers)
    if (app && pg == len / P) {
      u32x4 xk[NKS];
#pragma unroll
      for (int c = 0; c < NKS; ++c) xk[c] = *reinterpret_cast<const u32x4*>(&frow[8 * g + 32 * c]);
      fold_new_row(xk, len / P);
    }
  }
  const int p0 = (blockIdx.x * 4 + w) * 16;
  if (p0 < ncp) {
    float best[4] = {-INFINITY, -INFINITY, -INFINITY, -INFINITY};
    if (p0 < npages) {
      f32x4 acc[HB];
#pragma unroll
      for (int hb = 0; hb < HB; ++hb) acc[hb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int c = 0; c < NKS; ++c)
#pragma unroll
        for (int hb = 0; hb < HB; ++hb) acc[hb] = mfma_bf16_16x16x32(amx[c], qb[c][hb][lane], acc[hb]);
#pragma unroll
      for (int c = 0; c < NKS; ++c)
#pragma unroll
        for (int hb = 0; hb < HB; ++hb) acc[hb] = mfma_bf16_16x16x32(amn[c], qb[NKS + c][hb][lane], acc[hb]);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        float v = -INFINITY;
#pragma unroll
        for (int hb = 0; hb < HB; ++hb)
          if (16 * hb + c16 < G) v = fmaxf(v, acc[hb][r]);
        v = row16_max(v);
        best[r] = (p0 + 4 * g + r < npages) ? v : -INFINITY;
      }
    }
    if (c16 == 0) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int page = p0 + 4 * g + r;
        if (page < ncp) score[size_t(unit) * ncp + page] = best[r];
      }
    }
  }
}

// ------------------------------------------------------------------ wide-row scoring (latent 576)
// A group of 16 latent pages is 2 x 18 u32x4 of metadata per lane: too many
// registers to hold a second group as well, so blocks of one group per wave
// need two rounds of the GPU, the second starting only as the first drains.
// Here each wave scores NGW groups and streams them through one group's worth
// of registers: chunk r (16 pages x 32 columns) of group i is consumed by its
// MFMAs and its slot then reloads chunk r of group i + 1, so the wave keeps a
// group's worth of loads in flight across group boundaries.  The grid is two
// blocks per CU, each with an equal share of a unit's pages (groups dealt to
// its waves in turn), so every CU streams the same bytes in one round.  APP: the block holding the appended page folds the
// new row into that page's min / max while it stages q (the rebuild's last
// step), and the wave holding the page scores it again from the folded row.
template <int D, int HB, bool APP, int NGW>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2))) void quest_score_ring_kernel(
    const uint16_t* __restrict__ q, const uint16_t* kmin, const uint16_t* kmax,
    const int32_t* seq_len, float* score, int Hkv, int G, int P, int ncp, int cap, int ppb, QuestAppendArgs ap) {
  constexpr int NKS = D / 32, NCH = 2 * NKS;   // chunks per group: max rows k-steps 0.., then min rows
  __shared__ u32x4 qb[2 * NKS][HB][64];
  __shared__ __align__(16) uint16_t frow[APP ? 2 * D : 8];   // the appended page's folded max, min rows
  const int lane = threadIdx.x & 63, g = lane >> 4, c16 = lane & 15;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int unit = blockIdx.y, b = unit / Hkv, kvh = unit % Hkv;
  const int len = min(seq_len[b], cap);
  const bool app = APP && len < cap;                 // room for the new token
  const int new_len = app ? len + 1 : len;
  const int npages = min((new_len + P - 1) / P, ncp);
  const int plast = len / P;
  const bool fresh = len % P == 0;
  // the block's pages p_blk .. p_end - 1 in groups of 16; this wave's groups are
  // w, w + 4, ..  (its group gi starts at page p_blk + 16 (w + 4 gi))
  const int p_blk = blockIdx.x * ppb, p_end = min(ncp, p_blk + ppb);
  auto grp_page = [&](int gi) { return p_blk + 16 * (w + 4 * gi); };
  // chunk r of group gi; pages past the valid ones or past the block's own (the
  // next block's) read page 0, which stays in cache: unconditional loads keep the
  // wait counts exact; their bounds are masked or not stored
  const int p_load = min(npages, p_end);
  auto chunk_ptr = [&](int gi, int r) -> const uint16_t* {
    const int pg = grp_page(gi) + c16;
    const size_t row = size_t(unit) * ncp + (pg < p_load ? pg : 0);
    return (r < NKS ? kmax : kmin) + row * D + 8 * g + 32 * (r % NKS);
  };
  // q first (each 16-byte piece feeds both the q+ and the q- entry), then the
  // first group's chunks: all in flight together, and q's wait leaves the ring's
  // loads outstanding.  Unconditional loads (a clamped head, zeroed after) keep
  // the wait counts exact.
  const uint16_t* qg = q + (size_t(b) * Hkv * G + size_t(kvh) * G) * D;
  constexpr int QE = NKS * HB * 64, QR = QE / 256;
  static_assert(QE % 256 == 0, "q entries are dealt evenly to the block's threads");
  u32x4 qv[QR];
#pragma unroll
  for (int t = 0; t < QR; ++t) {
    const int idx = threadIdx.x + 256 * t;
    const int ln = idx & 63, hb = (idx >> 6) % HB, c = idx / (64 * HB);
    const int head = 16 * hb + (ln & 15);
    qv[t] = ld16(qg + size_t(min(head, G - 1)) * D + 32 * c + 8 * (ln >> 4));
  }
  __builtin_amdgcn_sched_barrier(0);   // q's loads stay ahead of the ring's
  u32x4 ring[NCH];
#pragma unroll
  for (int r = 0; r < NCH; ++r) ring[r] = ld16(chunk_ptr(0, r));
#pragma unroll
  for (int t = 0; t < QR; ++t) {
    const int idx = threadIdx.x + 256 * t;
    const int ln = idx & 63, hb = (idx >> 6) % HB, c = idx / (64 * HB);
    const int head = 16 * hb + (ln & 15);
    const u32x4 x = head < G ? qv[t] : u32x4{0, 0, 0, 0};
    u32x4 xp, xn;
    // q- keeps the halves whose sign bit is set, q+ the others
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
      const uint32_t sgn = ((x[jj] >> 15) & 1u) * 0xffffu | ((x[jj] >> 31) & 1u) * 0xffff0000u;
      xp[jj] = x[jj] & ~sgn;
      xn[jj] = x[jj] & sgn;
    }
    qb[c][hb][ln] = xp;
    qb[NKS + c][hb][ln] = xn;
  }
  const bool owner = app && p_blk <= plast && plast < p_end;   // the block holding the appended page
  if (APP && owner) {
    // the new K / V rows, and the appended page's min / max with the new row
    // folded in (the last step of the in-order rebuild), or the new row alone on
    // a fresh page; the stream still reads the old values of that page, whose
    // bound the wave holding it recomputes below
    const size_t urow = size_t(unit) * cap, mo = (size_t(unit) * ncp + plast) * D;
    for (int i = threadIdx.x; i < 2 * (D / 8); i += 256) {
      const bool isv = i >= D / 8;
      const int o = 8 * (isv ? i - D / 8 : i);
      if (!isv) {
        const u32x4 x = ld16(ap.k_new + size_t(unit) * D + o);
        *reinterpret_cast<u32x4*>(ap.k + (urow + len) * D + o) = x;
        const u32x4 omx = ld16(kmax + mo + o), omn = ld16(kmin + mo + o);
        u32x4 mx, mn;
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
          mx[jj] = bf16x2_fmin(fresh ? 0xff80ff80u : omx[jj], x[jj], true);    // -inf pair on a fresh page
          mn[jj] = bf16x2_fmin(fresh ? 0x7f807f80u : omn[jj], x[jj], false);   // +inf pair
        }
        *reinterpret_cast<u32x4*>(ap.kmax_w + mo + o) = mx;
        *reinterpret_cast<u32x4*>(ap.kmin_w + mo + o) = mn;
        *reinterpret_cast<u32x4*>(&frow[o]) = mx;
        *reinterpret_cast<u32x4*>(&frow[D + o]) = mn;
      } else if (ap.v != nullptr) {
        *reinterpret_cast<u32x4*>(ap.v + (urow + len) * D + o) = ld16(ap.v_new + size_t(unit) * D + o);
      }
    }
  }
  __syncthreads();
  // the group (-1: none) and lane row of this wave that hold the appended page
  const int rel = plast - p_blk;   // block group rel / 16 = wave (rel / 16) % 4, its group (rel / 16) / 4
  const int fold_gi = __builtin_amdgcn_readfirstlane((APP && owner && (rel >> 4) % 4 == w) ? (rel >> 4) / 4 : -1);
  const int fold_lane = rel & 15;
  f32x4 acc[HB];
  auto consume = [&](int r) {
#pragma unroll
    for (int hb = 0; hb < HB; ++hb) acc[hb] = mfma_bf16_16x16x32(ring[r], qb[r][hb][lane], acc[hb]);
  };
  auto finish = [&](int gi) {   // the group's bounds: maximum over the heads of each page
    const int p0 = grp_page(gi);
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      float v = -INFINITY;
#pragma unroll
      for (int hb = 0; hb < HB; ++hb)
        if (16 * hb + c16 < G) v = fmaxf(v, acc[hb][r]);
      v = row16_max(v);
      const int page = p0 + 4 * g + r;
      const bool stale = APP && fold_gi == gi && page == plast;   // scored again below
      if (c16 == 0 && page < p_end && !stale) score[size_t(unit) * ncp + page] = page < npages ? v : -INFINITY;
    }
  };
#pragma unroll
  for (int gi = 0; gi + 1 < NGW; ++gi) {   // the next group exists: its chunks load behind this one's
#pragma unroll
    for (int hb = 0; hb < HB; ++hb) acc[hb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int r = 0; r < NCH; ++r) {
      consume(r);
      ring[r] = ld16(chunk_ptr(gi + 1, r));
    }
    finish(gi);
  }
#pragma unroll
  for (int hb = 0; hb < HB; ++hb) acc[hb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int r = 0; r < NCH; ++r) consume(r);
  finish(NGW - 1);
  if (APP && fold_gi >= 0) {   // wave-uniform: the appended page's bound from its folded rows
#pragma unroll
    for (int hb = 0; hb < HB; ++hb) acc[hb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int r = 0; r < NCH; ++r) {
      const u32x4 x = c16 == fold_lane ? *reinterpret_cast<const u32x4*>(&frow[(r < NKS ? 0 : D) + 8 * g + 32 * (r % NKS)])
                                       : u32x4{0, 0, 0, 0};
#pragma unroll
      for (int hb = 0; hb < HB; ++hb) acc[hb] = mfma_bf16_16x16x32(x, qb[r][hb][lane], acc[hb]);
    }
    // row fold_lane sits in lanes g = fold_lane / 4, element fold_lane % 4
    float v = -INFINITY;
#pragma unroll
    for (int hb = 0; hb < HB; ++hb) {
      const f32x4 a4 = acc[hb];
      const float e = (fold_lane & 3) == 0 ? a4[0] : (fold_lane & 3) == 1 ? a4[1] : (fold_lane & 3) == 2 ? a4[2] : a4[3];
      if (16 * hb + c16 < G) v = fmaxf(v, e);
    }
    v = row16_max(v);
    if (g == (fold_lane >> 2) && c16 == 0) score[size_t(unit) * ncp + plast] = v;   // plast < npages
  }
}

// Grid of the wide-row kernel: two 4-wave blocks per CU (the q staging's LDS
// allows no more), split evenly over the units; at most 4 groups per wave.
static void quest_ring_grid(int ncp, int units, int* nbpu, int* ppb, int* ngw) {
  int n = std::max(1, std::min(512 / units, ceil_div(ncp, 16)));
  int p = ceil_div(ceil_div(ncp, n), 16) * 16;
  if (p > 4 * 4 * 16) p = 4 * 4 * 16;   // more blocks instead of more groups per wave
  *ppb = p;
  *nbpu = ceil_div(ncp, p);
  *ngw = ceil_div(p, 4 * 16);
}

template <bool APP>
static void launch_score_ring576(const se_cache& c, const void* q, const void* kmin, const void* kmax,
                                 const int32_t* seq_len, float* score, int P, int ncp, QuestAppendArgs ap,
                                 hipStream_t s) {
  const int units = c.batch * c.n_kv_heads, G = c.n_q_heads / c.n_kv_heads;
  int nbpu, ppb, ngw;
  quest_ring_grid(ncp, units, &nbpu, &ppb, &ngw);
#define SE_RG(NG) hipLaunchKernelGGL((quest_score_ring_kernel<576, 2, APP, NG>), dim3(nbpu, units), dim3(256), 0, s,   \
                                     (const uint16_t*)q, (const uint16_t*)kmin, (const uint16_t*)kmax, seq_len, score, \
                                     c.n_kv_heads, G, P, ncp, c.capacity, ppb, ap)
  if (ngw == 1) SE_RG(1);
  else if (ngw == 2) SE_RG(2);
  else if (ngw == 3) SE_RG(3);
  else SE_RG(4);
#undef SE_RG
}

// ------------------------------------------------------------------ top-k pages
// One block per unit: page scores -> ascending view.  Up to BLOCK * E pages
// the scores stay in registers (block_topk_reg); longer caches use the LDS /
// global-memory variant.
// APP (the fused decode call): pages are counted with the length after the
// append, and the block holding the last ticket of its batch row (counters[b],
// taken once the old length is read) stores the new length.
template <int BLOCK, int E, bool APP = false>
__global__ __launch_bounds__(BLOCK) void quest_topk_reg_kernel(
    const float* __restrict__ score, int32_t* seq_len, int32_t* __restrict__ view_idx,
    int32_t* __restrict__ view_len, int Hkv, int P, int n_cap_pages, int cap, int top_pages, int* counters) {
  __shared__ TopkRegShared sh;
  const int unit = blockIdx.x, b = unit / Hkv;
  const int len = min(seq_len[b], cap);
  const int new_len = (APP && len < cap) ? len + 1 : len;
  const int n = min((new_len + P - 1) / P, n_cap_pages);
  // APP: the row ticket is taken right after the score loads have been issued --
  // their addresses depend on the old length, so it has been read -- and its value
  // is looked at only at the end: the atomic's round trip overlaps the scores'
  // (the compiler waits for its return at once: the wave-aggregated atomic needs it)
  int ticket = 0;
  auto take_ticket = [&]() {
    if (APP && threadIdx.x == 0) {
      __atomic_signal_fence(__ATOMIC_SEQ_CST);
      ticket = __hip_atomic_fetch_add(counters + b, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __atomic_signal_fence(__ATOMIC_SEQ_CST);
    }
  };
  const float* su = score + size_t(unit) * n_cap_pages;
  const int kk = block_topk_reg<BLOCK, E>([&](int i) { return su[i]; }, n, top_pages,
                                          view_idx + size_t(unit) * top_pages, sh, take_ticket);
  if (threadIdx.x == 0) view_len[unit] = kk;
  if (APP && threadIdx.x == 0 && ticket == Hkv - 1) {   // every block of the row has read the old length
    if (new_len != len) seq_len[b] = new_len;
    ticket_reset(counters + b);
  }
}

template <int BLOCK>
__global__ __launch_bounds__(BLOCK) void quest_topk_block_kernel(
    const float* __restrict__ score, const int32_t* __restrict__ seq_len, int32_t* __restrict__ view_idx,
    int32_t* __restrict__ view_len, int Hkv, int P, int n_cap_pages, int cap, int top_pages) {
  __shared__ float s_lds[QUEST_TOPK_LDS];
  __shared__ TopkShared sh;
  const int unit = blockIdx.x, b = unit / Hkv;
  const int n = min((min(seq_len[b], cap) + P - 1) / P, n_cap_pages);
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

template <int D, int HB>
static void launch_score_mfma(const se_cache& c, const void* q, const void* kmin, const void* kmax,
                              const int32_t* seq_len, float* score, int P, int ncp, hipStream_t s) {
  const int units = c.batch * c.n_kv_heads, G = c.n_q_heads / c.n_kv_heads;
  // one group of 16 pages per wave: many small blocks keep the most metadata loads in flight
  hipLaunchKernelGGL((quest_score_mfma_kernel<D, HB, false>), dim3(ceil_div(ncp, 64), units), dim3(256), 0, s,
                     (const uint16_t*)q, (const uint16_t*)kmin, (const uint16_t*)kmax, seq_len, score, c.n_kv_heads,
                     G, P, ncp, c.capacity, QuestAppendArgs{});
}

// Largest page count of the fused call's register top-k (512 threads x 16 keys).
constexpr int QUEST_FUSED_MAX_PAGES = 512 * 16;

se_status launch_quest(const se_cache& c, const void* q, const void* kmin, const void* kmax,
                       const int32_t* seq_len, int page_size, int top_pages, int32_t* view_idx,
                       int32_t* view_len, float* page_score, void* ws, hipStream_t s) {
  const int units = c.batch * c.n_kv_heads, G = c.n_q_heads / c.n_kv_heads;
  const int ncp = ceil_div(c.capacity, page_size);
  float* score = page_score ? page_score : (float*)ws;
  bool done = false;
#define SE_MF(DD, HH) launch_score_mfma<DD, HH>(c, q, kmin, kmax, seq_len, score, page_size, ncp, s)
  if (c.dtype == SE_BF16) {
    done = true;
    if (c.d_k == 128 && G <= 16) SE_MF(128, 1);
    else if (c.d_k == 128 && G <= 32) SE_MF(128, 2);
    else if (c.d_k == 64 && G <= 16) SE_MF(64, 1);
    else if (c.d_k == 576 && G <= 32) launch_score_ring576<false>(c, q, kmin, kmax, seq_len, score, page_size, ncp, QuestAppendArgs{}, s);
    else done = false;
  }
#undef SE_MF
  if (!done) {
    const int ppb = 256 / G;
    dim3 grid(ceil_div(ncp, ppb), units);
    const size_t lds = (size_t(2) * G * c.d_k + 256) * sizeof(float);
    if (lds > 64 * 1024) return SE_ERR_UNSUPPORTED;
    if (c.dtype == SE_F32)
      hipLaunchKernelGGL(quest_score_vector_kernel<float>, grid, dim3(256), lds, s, (const float*)q,
                         (const float*)kmin, (const float*)kmax, seq_len, score, c.n_kv_heads, G, c.d_k,
                         page_size, ncp);
    else
      hipLaunchKernelGGL(quest_score_vector_kernel<bf16_t>, grid, dim3(256), lds, s, (const bf16_t*)q,
                         (const bf16_t*)kmin, (const bf16_t*)kmax, seq_len, score, c.n_kv_heads, G, c.d_k,
                         page_size, ncp);
  }
  if (hipGetLastError() != hipSuccess) return SE_ERR_HIP;
#define SE_TOPK(KERN, NT) hipLaunchKernelGGL(KERN, dim3(units), dim3(NT), 0, s, score, (int32_t*)seq_len, view_idx, \
                                          view_len, c.n_kv_heads, page_size, ncp, c.capacity, top_pages, nullptr)
  if (ncp <= 512 * 4) SE_TOPK((quest_topk_reg_kernel<512, 4>), 512);
  else if (ncp <= 512 * 8) SE_TOPK((quest_topk_reg_kernel<512, 8>), 512);
  else if (ncp <= 512 * 16) SE_TOPK((quest_topk_reg_kernel<512, 16>), 512);
  else hipLaunchKernelGGL(quest_topk_block_kernel<256>, dim3(units), dim3(256), 0, s, score, seq_len, view_idx,
                          view_len, c.n_kv_heads, page_size, ncp, c.capacity, top_pages);
#undef SE_TOPK
  return launch_status();
}

size_t quest_append_ws_bytes(const se_cache& c, int page_size) {
  const size_t ctr = size_t(c.batch) * sizeof(int);
  return (ctr + 255) / 256 * 256 + quest_ws_bytes(c, page_size, 0);
}

// The first launch of the fused Quest decode step (bf16 GQA with d_k 64 / 128 and
// G <= 16, or bf16 latent rows of 576 with G <= 32): the new rows, the appended
// page's min / max and every page's score (into page_score, else the workspace,
// after its batch-row counters); seq_len is left for the step's attention launch
// to update.
se_status launch_quest_append_scores(const se_cache& c, const void* q, void* k, void* v, const void* k_new,
                                     const void* v_new, const int32_t* seq_len, void* kmin, void* kmax, int page_size,
                                     float* page_score, void* ws, float** score_out, hipStream_t s) {
  const int units = c.batch * c.n_kv_heads, G = c.n_q_heads / c.n_kv_heads;
  const int ncp = ceil_div(c.capacity, page_size);
  const size_t ctr_bytes = (size_t(c.batch) * sizeof(int) + 255) / 256 * 256;
  float* score = page_score ? page_score : (float*)((char*)ws + ctr_bytes);
  QuestAppendArgs ap{};
  ap.k = (uint16_t*)k; ap.v = c.latent ? nullptr : (uint16_t*)v;
  ap.k_new = (const uint16_t*)k_new; ap.v_new = c.latent ? nullptr : (const uint16_t*)v_new;
  ap.kmin_w = (uint16_t*)kmin; ap.kmax_w = (uint16_t*)kmax;
  if (c.dtype == SE_BF16 && c.latent && c.d_k == 576 && G <= 32) {
    launch_score_ring576<true>(c, q, kmin, kmax, seq_len, score, page_size, ncp, ap, s);
    *score_out = score;
    return launch_status();
  }
  const dim3 grid(ceil_div(ncp, 64), units);
#define SE_AP(DD) hipLaunchKernelGGL((quest_score_mfma_kernel<DD, 1, true>), grid, dim3(256), 0, s, (const uint16_t*)q, \
                                     (const uint16_t*)kmin, (const uint16_t*)kmax, seq_len, score, c.n_kv_heads, G,  \
                                     page_size, ncp, c.capacity, ap)
  if (c.dtype != SE_BF16 || c.latent || G > 16) return SE_ERR_UNSUPPORTED;
  if (c.d_k == 128) SE_AP(128);
  else if (c.d_k == 64) SE_AP(64);
  else return SE_ERR_UNSUPPORTED;
#undef SE_AP
  *score_out = score;
  return launch_status();
}

// The first launch of the fused Quest decode step over FP8 rows (GQA, d_k 64 / 128,
// G <= 16): the new rows quantized into codes and scale bytes, the stored K values
// folded into the appended page's min / max, and every page's score; seq_len is
// left for the step's attention launch to update.
se_status launch_quest_fp8_append_scores(const se_cache& c, const void* q, void* kq, void* vq, void* ks, void* vs,
                                         const void* k_new, const void* v_new, const int32_t* seq_len, void* kmin,
                                         void* kmax, int page_size, float* page_score, void* ws, float** score_out,
                                         hipStream_t s) {
  const int units = c.batch * c.n_kv_heads, G = c.n_q_heads / c.n_kv_heads;
  const int ncp = ceil_div(c.capacity, page_size);
  const size_t ctr_bytes = (size_t(c.batch) * sizeof(int) + 255) / 256 * 256;
  float* score = page_score ? page_score : (float*)((char*)ws + ctr_bytes);
  QuestAppendArgs ap{};
  ap.k_new = (const uint16_t*)k_new; ap.v_new = (const uint16_t*)v_new;
  ap.kmin_w = (uint16_t*)kmin; ap.kmax_w = (uint16_t*)kmax;
  ap.kq = (uint8_t*)kq; ap.vq = (uint8_t*)vq; ap.ks = (uint8_t*)ks; ap.vs = (uint8_t*)vs;
  if (c.dtype != SE_BF16 || c.latent || G > 16) return SE_ERR_UNSUPPORTED;
  const dim3 grid(ceil_div(ncp, 64), units);
#define SE_AP(DD) hipLaunchKernelGGL((quest_score_mfma_kernel<DD, 1, 2>), grid, dim3(256), 0, s, (const uint16_t*)q, \
                                     (const uint16_t*)kmin, (const uint16_t*)kmax, seq_len, score, c.n_kv_heads, G, \
                                     page_size, ncp, c.capacity, ap)
  if (c.d_k == 128) SE_AP(128);
  else if (c.d_k == 64) SE_AP(64);
  else return SE_ERR_UNSUPPORTED;
#undef SE_AP
  *score_out = score;
  return launch_status();
}

// Two launches: append + page scores, then top-k + the new seq_len.
se_status launch_quest_append(const se_cache& c, const void* q, void* k, void* v, const void* k_new,
                              const void* v_new, int32_t* seq_len, void* kmin, void* kmax, int page_size,
                              int top_pages, int32_t* view_idx, int32_t* view_len, float* page_score, void* ws,
                              hipStream_t s) {
  const int units = c.batch * c.n_kv_heads, G = c.n_q_heads / c.n_kv_heads;
  const int ncp = ceil_div(c.capacity, page_size);
  const size_t ctr_bytes = (size_t(c.batch) * sizeof(int) + 255) / 256 * 256;
  float* score = page_score ? page_score : (float*)((char*)ws + ctr_bytes);
  int* counters = (int*)ws;
  QuestAppendArgs ap{};
  ap.k = (uint16_t*)k; ap.v = c.latent ? nullptr : (uint16_t*)v;
  ap.k_new = (const uint16_t*)k_new; ap.v_new = c.latent ? nullptr : (const uint16_t*)v_new;
  ap.kmin_w = (uint16_t*)kmin; ap.kmax_w = (uint16_t*)kmax;
  bool fused = c.dtype == SE_BF16 && ncp <= QUEST_FUSED_MAX_PAGES;
  if (fused) {
    const dim3 grid(ceil_div(ncp, 64), units);
#define SE_AP(DD, HH) hipLaunchKernelGGL((quest_score_mfma_kernel<DD, HH, true>), grid, dim3(256), 0, s,           \
                                         (const uint16_t*)q, (const uint16_t*)kmin, (const uint16_t*)kmax, seq_len, \
                                         score, c.n_kv_heads, G, page_size, ncp, c.capacity, ap)
    if (c.d_k == 128 && G <= 16) SE_AP(128, 1);
    else if (c.d_k == 128 && G <= 32) SE_AP(128, 2);
    else if (c.d_k == 64 && G <= 16) SE_AP(64, 1);
    else if (c.d_k == 576 && G <= 32) launch_score_ring576<true>(c, q, kmin, kmax, seq_len, score, page_size, ncp, ap, s);
    else fused = false;
#undef SE_AP
  }
  if (!fused) {   // other shapes: the separate append and selection launches (same results)
    se_status st = launch_kv_append_meta(c, k, v, k_new, v_new, nullptr, seq_len, kmin, kmax, page_size, s);
    if (st != SE_OK) return st;
    return launch_quest(c, q, kmin, kmax, seq_len, page_size, top_pages, view_idx, view_len, page_score,
                        (char*)ws + ctr_bytes, s);
  }
  if (hipGetLastError() != hipSuccess) return SE_ERR_HIP;
#define SE_TK(EE) hipLaunchKernelGGL((quest_topk_reg_kernel<512, EE, true>), dim3(units), dim3(512), 0, s, score, \
                                     seq_len, view_idx, view_len, c.n_kv_heads, page_size, ncp, c.capacity,      \
                                     top_pages, counters)
  if (ncp <= 512 * 4) SE_TK(4);
  else if (ncp <= 512 * 8) SE_TK(8);
  else SE_TK(16);
#undef SE_TK
  return launch_status();
}

}  // namespace se
