// SnapKV prefill-end eviction: observation-window votes, max-pool, top-k, compaction.
//
// tokendh.com explainer, section "把边界划在'生命周期'上": at its hook SnapKV
// looks at how the last few prompt tokens attend over the history, keeps the
// important part and physically deletes the rest.  Here the window rows are
// the G x W queries (head h, window index i) at positions L - W + i; row r's
// softmax runs causally over keys 0 .. L - W + i; a history key's vote is the
// sum of the rows' weights on it; votes are max-pooled (odd width, stride 1);
// the best budget - W pooled positions (ties to the lower position) and the
// window are kept, ascending, and their K / V rows are copied out.
//
// The window scores are a dense contraction (G x W rows share every key), so
// bf16 caches score them on MFMA in two passes over K: pass A forms each row's
// log-sum-exp (split over key chunks, then merged), pass B sums the softmax
// weights per key.  fp32 caches use vector kernels.
#include <type_traits>

#include "se_internal.hpp"
#include "mfma_util.hpp"

namespace se {

constexpr float SK_LOG2E = 1.4426950408889634f;
// keys per block in the MFMA passes: chosen per call (snap_chunk_keys) between these;
// the maximum is what pass B's per-wave key sums leave of the LDS at three blocks per CU
constexpr int SK_CHUNK_MAX = 1104;
constexpr int SK_CHUNK_MIN = 512;
constexpr float SK_MARGIN = 8.f;      // lazy running-max margin (log2 units)
constexpr int SK_KT = 64;             // keys per LDS tile in the MFMA passes

struct SelState { uint32_t prefix, mask; int r, done; };   // per-unit radix-select state

struct SnapArgs {
  const void* q; const void* k; const void* v;
  void* k_out; void* v_out;
  int32_t* kept; float* votes; float* pooled; float* part; float* lse2; int32_t* out_len;
  uint32_t* sel_hist; SelState* sel_state; int32_t* sel_counts;   // multi-block select
  int B, Hq, Hkv, G, D, cap, out_cap, L, W, R, pool, budget, nchunks, chunk, dtype;
  float sc2;   // scale * log2(e)
};

// The lazy running max of pass A: moved (and the sum rescaled) only when a block's
// max exceeds it by more than the margin.  The branch is taken by the whole wave when
// any lane moves (rare once the rows' maxima settle), so no lane's registers are
// shuffled through divergent control flow; lanes that do not move keep m and l.
__device__ __forceinline__ void sk_grow(float bm, float& m, float& l) {
  const bool grow = bm > m + SK_MARGIN;
  if (__ballot(grow) != 0) {
    const float f = (m == -INFINITY) ? 0.f : ex2(m - bm);
    l = grow ? l * f : l;
    m = grow ? bm : m;
  }
}

// ------------------------------------------------------------------ MFMA passes (bf16)
// grid (chunks, units); 4 waves, each owning NRB 16-row blocks of the R = 64 * NRB rows.
// Pass A takes S^T[key][row] = K[key] . Q[row]: A = 16 key rows (lane: key c16,
// dims 32c + 8g..), B = Q^T of one 16-row block (lane: row c16, same dims), so
// lane (g, c16) holds keys 4g..4g+3 of row c16 and a row's statistics stay in
// four lanes.  Pass B swaps the operands: lane (g, c16) holds rows 4g..4g+3 of
// key c16, and a key's vote stays in four lanes.
template <int D, int NRB, bool PASS_B>
// three waves per SIMD (three blocks per CU): pass A's pipelined body needs 176
// registers left free and so would run two, for four spilled registers at three
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(3))) void snap_mfma_kernel(SnapArgs a) {
  constexpr int NKS = D / 32, PITCH = D + 8, CH = D / 8, TPT = SK_KT * CH / 256;
  __shared__ __align__(16) uint16_t kt[2][SK_KT][PITCH];
  __shared__ float vsum[PASS_B ? 4 : 1][SK_CHUNK_MAX / 16][16];   // pass B: per-wave key sums of each 16-key block
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, g = lane >> 4, c16 = lane & 15;
  const int unit = blockIdx.y, chunk = blockIdx.x;
  const int b = unit / a.Hkv, kvh = unit % a.Hkv;
  const int n_hist = a.L - a.W;
  const int kend = PASS_B ? n_hist : a.L;          // pass B scores history keys only
  const int k0 = chunk * a.chunk, k1 = min(kend, k0 + a.chunk);
  const uint16_t* ku = (const uint16_t*)a.k + size_t(unit) * a.cap * D;
  const uint16_t* qu = (const uint16_t*)a.q + (size_t(b) * a.Hq + size_t(kvh) * a.G) * a.W * D;
  // Q operand of this wave's row blocks
  u32x4 qv[NRB][NKS];
  int rowpos[NRB];
  float nlse[NRB][4];   // pass B: -lse2 of rows 4g + i of each block (keys in the N dimension)
#pragma unroll
  for (int rb = 0; rb < NRB; ++rb) {
    const int row = (w * NRB + rb) * 16 + c16;
    rowpos[rb] = a.L - a.W + row % a.W;
#pragma unroll
    for (int c = 0; c < NKS; ++c) qv[rb][c] = ld16(qu + size_t(row) * D + 32 * c + 8 * g);
#pragma unroll
    for (int i = 0; i < 4; ++i)
      nlse[rb][i] = PASS_B ? -a.lse2[size_t(unit) * a.R + (w * NRB + rb) * 16 + 4 * g + i] : 0.f;
  }
  // q's and lse's loads stay ahead of the first K tile's: the wait that tile's LDS
  // store takes then covers them, and no wait inside the tile loop is left waiting for
  // them (or, behind them in the in-order count, for the next tile's prefetch)
  __builtin_amdgcn_sched_barrier(0);
  float m[NRB], l[NRB];
#pragma unroll
  for (int rb = 0; rb < NRB; ++rb) { m[rb] = -INFINITY; l[rb] = 0.f; }

  const int nblk = (k1 - k0 + 15) / 16;
  // blocks below `plain` hold no key past k1 and no window key, so no row masks any of them
  const int plain = (min(k1, n_hist) - k0) / 16;
  // K tiles of SK_KT keys go through double-buffered LDS, loaded by the whole block
  // one tile ahead (keys past k1 are clamped rows, masked below)
  const int ntile = (k1 - k0 + SK_KT - 1) / SK_KT;   // >= 1: every chunk of the grid starts below k1
  u32x4 stage[TPT];
  auto fetch = [&](int t) {
#pragma unroll
    for (int i = 0; i < TPT; ++i) {
      const int e = threadIdx.x + 256 * i;
      const int key = min(k0 + t * SK_KT + e / CH, a.cap - 1);
      stage[i] = ld16(ku + size_t(key) * D + 8 * (e % CH));
    }
  };
  auto put = [&](int buf) {
#pragma unroll
    for (int i = 0; i < TPT; ++i) {
      const int e = threadIdx.x + 256 * i;
      *reinterpret_cast<u32x4*>(&kt[buf][e / CH][8 * (e % CH)]) = stage[i];
    }
  };
  fetch(0);
  put(0);
  __syncthreads();
  // One 16-key block of a tile.  PLAIN (pass A): no key of the block is past k1 or
  // past any row's position, so no mask is formed.
  auto key_block = [&](int buf, int sb, int blk, auto plain_c) {
    constexpr bool PLAIN = decltype(plain_c)::value;
    u32x4 kc[NKS];
#pragma unroll
    for (int c = 0; c < NKS; ++c) kc[c] = *reinterpret_cast<const u32x4*>(&kt[buf][16 * sb + c16][8 * g + 32 * c]);
    const int kb = k0 + blk * 16;
    if constexpr (!PASS_B) {
      // S^T[key][row]: lane (g, c16) holds keys kb + 4g + i of row c16
#pragma unroll
      for (int rb = 0; rb < NRB; ++rb) {
        f32x4 s = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int c = 0; c < NKS; ++c) s = mfma_bf16_16x16x32(kc[c], qv[rb][c], s);
        if constexpr (PLAIN) {
          // the block max scaled once (sc2 > 0 and rounding is monotonic, so it equals
          // the max of the scaled logits) and each term as one fma
          const float bm = fmaxf(fmaxf(s[0], s[1]), fmaxf(s[2], s[3])) * a.sc2;
          sk_grow(bm, m[rb], l[rb]);
          const float nref = m[rb] == -INFINITY ? 0.f : -m[rb];
#pragma unroll
          for (int i = 0; i < 4; ++i) l[rb] += ex2(fmaf(s[i], a.sc2, nref));
        } else {
          float v[4];
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int key = kb + 4 * g + i;
            v[i] = key < k1 && key <= rowpos[rb] ? s[i] * a.sc2 : -INFINITY;
          }
          const float bm = fmaxf(fmaxf(v[0], v[1]), fmaxf(v[2], v[3]));
          sk_grow(bm, m[rb], l[rb]);
          const float mref = m[rb] == -INFINITY ? 0.f : m[rb];
#pragma unroll
          for (int i = 0; i < 4; ++i) l[rb] += ex2(v[i] - mref);
        }
      }
    } else {
      // S[row][key]: lane (g, c16) holds rows 4g + i of key kb + c16, so a key's sum
      // over the wave's rows stays in its lane until two exchanges across g.
      // History keys precede every window row: only keys past k1 are dropped.
      float vote = 0.f;
#pragma unroll
      for (int rb = 0; rb < NRB; ++rb) {
        f32x4 s = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int c = 0; c < NKS; ++c) s = mfma_bf16_16x16x32(qv[rb][c], kc[c], s);
#pragma unroll
        for (int i = 0; i < 4; ++i) vote += ex2(fmaf(s[i], a.sc2, nlse[rb][i]));
      }
      vote = rows4_sum(vote);
      if (g == 0) vsum[w][blk][c16] = kb + c16 < k1 ? vote : 0.f;
    }
  };
  // A tile whose four blocks all need no mask (and exist): one straight-line software
  // pipeline over its (16-key block, row block) pairs, the next pair's MFMAs issued
  // before this pair's exps (the passes are bound by the vector ALU: one exp2 and two
  // to three other operations per score), the next key block's operands read from
  // LDS a block ahead.
  auto plain_tile = [&](int buf, int t) {
    constexpr int NSB = SK_KT / 16, NP = NSB * NRB;
    u32x4 kc[2][NKS];
    auto rd = [&](int sb) {
#pragma unroll
      for (int c = 0; c < NKS; ++c)
        kc[sb & 1][c] = *reinterpret_cast<const u32x4*>(&kt[buf][16 * sb + c16][8 * g + 32 * c]);
    };
    auto mm = [&](int p) {
      const int sb = p / NRB, rb = p % NRB;
      f32x4 r = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int c = 0; c < NKS; ++c)
        r = PASS_B ? mfma_bf16_16x16x32(qv[rb][c], kc[sb & 1][c], r) : mfma_bf16_16x16x32(kc[sb & 1][c], qv[rb][c], r);
      return r;
    };
    // pass A: raw score above which a key moves a row's running max, (m + margin) / sc2
    float thr[NRB];
    const float inv_sc2 = 1.f / a.sc2;
#pragma unroll
    for (int rb = 0; rb < NRB; ++rb) thr[rb] = (m[rb] + SK_MARGIN) * inv_sc2;
    float vote = 0.f;
    rd(0);
    f32x4 sc = mm(0);
#pragma unroll
    for (int p = 0; p < NP; ++p) {
      const int sb = p / NRB, rb = p % NRB;
      if (rb == 0 && sb + 1 < NSB) rd(sb + 1);
      f32x4 sn = sc;
      if (p + 1 < NP) sn = mm(p + 1);
      if constexpr (!PASS_B) {
        // the lazy running max (the rule sk_grow applies), tested on the raw scores
        const bool up = (sc[0] > thr[rb]) | (sc[1] > thr[rb]) | (sc[2] > thr[rb]) | (sc[3] > thr[rb]);
        if (__ballot(up) != 0) {
          const float bm = fmaxf(fmaxf(sc[0], sc[1]), fmaxf(sc[2], sc[3])) * a.sc2;
          l[rb] = up ? (m[rb] == -INFINITY ? 0.f : l[rb] * ex2(m[rb] - bm)) : l[rb];
          thr[rb] = up ? (bm + SK_MARGIN) * inv_sc2 : thr[rb];
          m[rb] = up ? bm : m[rb];
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) l[rb] += ex2(fmaf(sc[i], a.sc2, -m[rb]));
        // keeps the sum here: left free, the compiler sinks it to the row block's next
        // pair and holds the scores of the pairs between in registers
        asm volatile("" : "+v"(l[rb]));
      } else {
#pragma unroll
        for (int i = 0; i < 4; ++i) vote += ex2(fmaf(sc[i], a.sc2, nlse[rb][i]));
        if (rb == NRB - 1) {
          const float v = rows4_sum(vote);
          if (g == 0) vsum[w][t * NSB + sb][c16] = v;
          vote = 0.f;
        }
      }
      sc = sn;
    }
  };
  using Plain = std::integral_constant<bool, true>;
  using Masked = std::integral_constant<bool, false>;
  for (int t = 0; t < ntile; ++t) {
    const int buf = t & 1;
    if (t + 1 < ntile) fetch(t + 1);
    // tiles whose four blocks all need no mask (and exist) take the pipelined body;
    // the chunk's last tiles take the general one (uniform across the block)
    if ((t + 1) * (SK_KT / 16) <= (PASS_B ? nblk : plain)) {
      plain_tile(buf, t);
    } else {
#pragma unroll
      for (int sb = 0; sb < SK_KT / 16; ++sb) {
        const int blk = t * (SK_KT / 16) + sb;
        if (blk >= nblk) break;
        if (PASS_B || blk < plain) key_block(buf, sb, blk, Plain{});
        else key_block(buf, sb, blk, Masked{});
      }
    }
    if (t + 1 < ntile) put(buf ^ 1);
    __syncthreads();
  }
  if (!PASS_B) {
    // merge the 4 lanes of each row (g = 0..3), then write the chunk's partial
#pragma unroll
    for (int rb = 0; rb < NRB; ++rb) {
      float mm = m[rb];
      mm = rows4_max(mm);
      float ll = (m[rb] == -INFINITY) ? 0.f : l[rb] * ex2(m[rb] - mm);
      ll = rows4_sum(ll);
      if (g == 0) {
        const int row = (w * NRB + rb) * 16 + c16;
        float* p = a.part + ((size_t(unit) * a.nchunks + chunk) * a.R + row) * 2;
        p[0] = mm;
        p[1] = ll;
      }
    }
  } else {
    __syncthreads();
    for (int j = threadIdx.x; j < k1 - k0; j += 256) {
      const float t = vsum[0][j / 16][j % 16] + vsum[1][j / 16][j % 16] + vsum[2][j / 16][j % 16] +
                      vsum[3][j / 16][j % 16];
      a.votes[size_t(unit) * n_hist + k0 + j] = t;
    }
  }
}

// Eight threads per (unit, row): each folds every eighth chunk partial into a
// running (max, sum) with all of its loads in flight together, then the eight
// combine by lane exchange into the row's log2-sum-exp2.
constexpr int SK_MERGE_LANES = 8;
__global__ __launch_bounds__(256) void snap_lse_merge_kernel(SnapArgs a) {
  const int gid = blockIdx.x * blockDim.x + threadIdx.x;
  const int idx = gid / SK_MERGE_LANES, part = gid % SK_MERGE_LANES;
  const bool live = idx < a.B * a.Hkv * a.R;   // whole groups of eight share this (lanes stay active)
  const int unit = live ? idx / a.R : 0, row = live ? idx % a.R : 0;
  float M = -INFINITY, S = 0.f;
  if (live) {
    constexpr int BATCH = 8;
    for (int c0 = part; c0 < a.nchunks; c0 += SK_MERGE_LANES * BATCH) {
      float mb[BATCH], lb[BATCH];
#pragma unroll
      for (int j = 0; j < BATCH; ++j) {
        const int c = min(c0 + j * SK_MERGE_LANES, a.nchunks - 1);
        const float* p = a.part + ((size_t(unit) * a.nchunks + c) * a.R + row) * 2;
        mb[j] = c0 + j * SK_MERGE_LANES < a.nchunks ? p[0] : -INFINITY;
        lb[j] = p[1];
      }
      float Mb = M;
#pragma unroll
      for (int j = 0; j < BATCH; ++j) Mb = fmaxf(Mb, mb[j]);
      if (Mb == -INFINITY) continue;
      S = (M == -INFINITY) ? 0.f : S * ex2(M - Mb);
#pragma unroll
      for (int j = 0; j < BATCH; ++j)
        if (mb[j] != -INFINITY) S += lb[j] * ex2(mb[j] - Mb);
      M = Mb;
    }
  }
#pragma unroll
  for (int o = 1; o < SK_MERGE_LANES; o <<= 1) {
    const float Mo = __shfl_xor(M, o, 64), So = __shfl_xor(S, o, 64);
    const float Mn = fmaxf(M, Mo);
    if (Mn != -INFINITY) {
      S = (M == -INFINITY ? 0.f : S * ex2(M - Mn)) + (Mo == -INFINITY ? 0.f : So * ex2(Mo - Mn));
      M = Mn;
    }
  }
  if (live && part == 0) a.lse2[idx] = M + log2f(S);
}

// ------------------------------------------------------------------ vector passes (any dtype)
template <typename T>
__global__ __launch_bounds__(256) void snap_vec_lse_kernel(SnapArgs a) {
  extern __shared__ float qrow[];   // [D]
  __shared__ float rm[4], rl[4];
  const int row = blockIdx.x, unit = blockIdx.y;
  const int b = unit / a.Hkv, kvh = unit % a.Hkv, D = a.D;
  const T* qu = (const T*)a.q + ((size_t(b) * a.Hq + size_t(kvh) * a.G) * a.W + row) * D;
  const T* ku = (const T*)a.k + size_t(unit) * a.cap * D;
  for (int d = threadIdx.x; d < D; d += 256) qrow[d] = to_f32(qu[d]);
  __syncthreads();
  const int pos = a.L - a.W + row % a.W;
  float m = -INFINITY, l = 0.f;
  for (int j = threadIdx.x; j <= pos; j += 256) {
    float dot = 0.f;
    for (int d = 0; d < D; ++d) dot += qrow[d] * to_f32(ku[size_t(j) * D + d]);
    const float s = dot * a.sc2;
    if (s > m) { l = l * ex2(m - s); m = s; }
    l += ex2(s - m);
  }
  const float mw = wave_max(m);
  l = (m == -INFINITY) ? 0.f : l * ex2(m - mw);
  l = wave_sum(l);
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  if (lane == 0) { rm[w] = mw; rl[w] = l; }
  __syncthreads();
  if (threadIdx.x == 0) {
    float M = fmaxf(fmaxf(rm[0], rm[1]), fmaxf(rm[2], rm[3])), S = 0.f;
    for (int i = 0; i < 4; ++i)
      if (rm[i] != -INFINITY) S += rl[i] * ex2(rm[i] - M);
    a.lse2[size_t(unit) * a.R + row] = M + log2f(S);
  }
}

template <typename T>
__global__ __launch_bounds__(256) void snap_vec_vote_kernel(SnapArgs a) {
  extern __shared__ float qs[];   // [R][D]
  const int unit = blockIdx.y, b = unit / a.Hkv, kvh = unit % a.Hkv, D = a.D;
  const T* qu = (const T*)a.q + (size_t(b) * a.Hq + size_t(kvh) * a.G) * a.W * D;
  const T* ku = (const T*)a.k + size_t(unit) * a.cap * D;
  for (int i = threadIdx.x; i < a.R * D; i += 256) qs[i] = to_f32(qu[i]);
  __syncthreads();
  const int n_hist = a.L - a.W;
  const int j = blockIdx.x * 256 + threadIdx.x;
  if (j >= n_hist) return;
  float vote = 0.f;
  for (int r = 0; r < a.R; ++r) {
    float dot = 0.f;
    for (int d = 0; d < D; ++d) dot += qs[r * D + d] * to_f32(ku[size_t(j) * D + d]);
    vote += ex2(dot * a.sc2 - a.lse2[size_t(unit) * a.R + r]);
  }
  a.votes[size_t(unit) * n_hist + j] = vote;
}

// ------------------------------------------------------------------ pool, select, gather
// grid (tiles of SK_POOL_T votes, units): the tile and its halo are staged in LDS.
constexpr int SK_POOL_T = 1024, SK_POOL_MAXR = 64;   // pool widths up to 129 (checked by the API)
__global__ __launch_bounds__(256) void snap_pool_kernel(SnapArgs a) {
  __shared__ float v_s[SK_POOL_T + 2 * SK_POOL_MAXR];
  const int unit = blockIdx.y, n = a.L - a.W, r = a.pool / 2;
  const float* v = a.votes + size_t(unit) * n;
  const int t0 = blockIdx.x * SK_POOL_T;
  for (int i = threadIdx.x; i < SK_POOL_T + 2 * r; i += 256) {
    const int j = t0 - r + i;
    v_s[i] = (j >= 0 && j < n) ? v[j] : -INFINITY;
  }
  __syncthreads();
  for (int i = threadIdx.x; i < SK_POOL_T; i += 256) {
    const int j = t0 + i;
    if (j >= n) break;
    float mx = -INFINITY;
    for (int d = 0; d <= 2 * r; ++d) mx = fmaxf(mx, v_s[i + d]);
    a.pooled[size_t(unit) * n + j] = mx;
  }
}

// ------------------------------------------------------------------ multi-block select
// The kept history positions are the k = budget - W largest pooled votes (ties
// to the lower position), in ascending order.  With n = L - W in the hundred
// thousands per unit, the selection is spread over SK_SEL_CH-element slices
// of every unit: three radix passes on the 32-bit ordered vote keys (digits of
// 11, 11 and 10 bits) each count digits in a per-block LDS histogram that is
// added into a per-unit global histogram, and a per-unit block finds the digit
// holding the k-th key (it also zeroes the global histogram again).  The kept
// set is every key above the resolved prefix plus the first r keys of its
// bucket in index order; a count pass and a write pass place them.
constexpr int SK_SEL_BLOCK = 256, SK_SEL_PER = 16, SK_SEL_CH = SK_SEL_BLOCK * SK_SEL_PER;
constexpr int SK_SEL_BINS = 2048;

__device__ __forceinline__ int sel_shift(int pass) { return pass == 0 ? 21 : pass == 1 ? 10 : 0; }
__device__ __forceinline__ uint32_t sel_dmask(int pass) { return pass == 2 ? 0x3ffu : 0x7ffu; }

// grid (slices, units)
__global__ __launch_bounds__(SK_SEL_BLOCK) void snap_sel_hist_kernel(SnapArgs a, int pass) {
  __shared__ uint32_t h[SK_SEL_BINS];
  const int unit = blockIdx.y, n = a.L - a.W;
  uint32_t prefix = 0u, mask = 0u;
  if (pass > 0) {
    const SelState st = a.sel_state[unit];
    if (st.done) return;
    prefix = st.prefix;
    mask = st.mask;
  }
  for (int i = threadIdx.x; i < SK_SEL_BINS; i += SK_SEL_BLOCK) h[i] = 0u;
  __syncthreads();
  const float* pv = a.pooled + size_t(unit) * n;
  const int shift = sel_shift(pass);
  const uint32_t dm = sel_dmask(pass);
  const int i0 = blockIdx.x * SK_SEL_CH;
#pragma unroll 4
  for (int j = 0; j < SK_SEL_PER; ++j) {
    const int i = i0 + j * SK_SEL_BLOCK + threadIdx.x;
    if (i < n) {
      const uint32_t key = ordered_bits(pv[i]);
      if ((key & mask) == prefix) atomicAdd(&h[(key >> shift) & dm], 1u);
    }
  }
  __syncthreads();
  uint32_t* gh = a.sel_hist + size_t(unit) * SK_SEL_BINS;
  for (int i = threadIdx.x; i < SK_SEL_BINS; i += SK_SEL_BLOCK)
    if (h[i] != 0u) atomicAdd(&gh[i], h[i]);
}

// grid (units): finds the digit holding the r-th largest remaining key; zeroes the histogram.
__global__ __launch_bounds__(SK_SEL_BLOCK) void snap_sel_find_kernel(SnapArgs a, int pass, int kk) {
  __shared__ int scan_tmp[SK_SEL_BLOCK / WAVE];
  __shared__ int res[3];
  const int unit = blockIdx.x, n = a.L - a.W;
  SelState st;
  if (pass == 0) {
    st.prefix = 0u; st.mask = 0u; st.r = kk;
    st.done = (kk <= 0 || kk >= n) ? 1 : 0;
  } else {
    st = a.sel_state[unit];
  }
  uint32_t* gh = a.sel_hist + size_t(unit) * SK_SEL_BINS;
  // thread t owns digits 2047 - 8t .. 2040 - 8t (descending)
  constexpr int PER = SK_SEL_BINS / SK_SEL_BLOCK;
  int c[PER];
  int own = 0;
#pragma unroll
  for (int j = 0; j < PER; ++j) {
    const int d = SK_SEL_BINS - 1 - PER * threadIdx.x - j;
    c[j] = int(gh[d]);
    gh[d] = 0u;
    own += c[j];
  }
  if (st.done) {
    if (pass == 0 && threadIdx.x == 0) a.sel_state[unit] = st;
    return;
  }
  int total;
  const int incl = block_excl_scan<SK_SEL_BLOCK>(own, scan_tmp, &total) + own;
  int above = incl - own;
  if (above < st.r && st.r <= incl) {
#pragma unroll
    for (int j = 0; j < PER; ++j) {
      if (above + c[j] >= st.r) {
        res[0] = SK_SEL_BINS - 1 - PER * threadIdx.x - j;
        res[1] = st.r - above;
        res[2] = c[j];
        break;
      }
      above += c[j];
    }
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    const int shift = sel_shift(pass);
    st.prefix |= uint32_t(res[0]) << shift;
    st.mask |= sel_dmask(pass) << shift;
    st.r = res[1];
    st.done = (res[2] == res[1] || pass == 2) ? 1 : 0;
    a.sel_state[unit] = st;
  }
}

__device__ __forceinline__ void sel_classify(uint32_t key, const SelState& st, bool& above, bool& bucket) {
  const uint32_t km = key & st.mask;
  above = km > st.prefix;
  bucket = km == st.prefix;
}

// grid (slices, units): per-slice counts of keys above the prefix and in its bucket;
// slice 0 also writes the window entries, the -1 padding and out_len.
__global__ __launch_bounds__(SK_SEL_BLOCK) void snap_sel_count_kernel(SnapArgs a, int kk) {
  __shared__ int red[2][SK_SEL_BLOCK / WAVE];
  const int unit = blockIdx.y, n = a.L - a.W;
  const SelState st = a.sel_state[unit];
  const float* pv = a.pooled + size_t(unit) * n;
  const int i0 = blockIdx.x * SK_SEL_CH;
  int na = 0, nb = 0;
  for (int j = 0; j < SK_SEL_PER; ++j) {
    const int i = i0 + j * SK_SEL_BLOCK + threadIdx.x;
    if (i < n) {
      bool ab, bu;
      sel_classify(ordered_bits(pv[i]), st, ab, bu);
      na += ab;
      nb += bu;
    }
  }
  na = wave_sum_i(na);
  nb = wave_sum_i(nb);
  const int lane = threadIdx.x & (WAVE - 1), w = threadIdx.x / WAVE;
  if (lane == 0) { red[0][w] = na; red[1][w] = nb; }
  __syncthreads();
  if (threadIdx.x == 0) {
    int ta = 0, tb = 0;
    for (int i = 0; i < SK_SEL_BLOCK / WAVE; ++i) { ta += red[0][i]; tb += red[1][i]; }
    a.sel_counts[(size_t(unit) * gridDim.x + blockIdx.x) * 2] = ta;
    a.sel_counts[(size_t(unit) * gridDim.x + blockIdx.x) * 2 + 1] = tb;
  }
  if (blockIdx.x == 0) {
    int32_t* kept = a.kept + size_t(unit) * a.budget;
    for (int i = threadIdx.x; i < a.W; i += SK_SEL_BLOCK) kept[kk + i] = n + i;
    for (int i = kk + a.W + threadIdx.x; i < a.budget; i += SK_SEL_BLOCK) kept[i] = -1;
    if (threadIdx.x == 0 && unit % a.Hkv == 0 && a.out_len != nullptr) a.out_len[unit / a.Hkv] = kk + a.W;
  }
}

// grid (slices, units): writes the kept positions of the slice in ascending order.
// Thread t handles the contiguous elements [i0 + 16 t, i0 + 16 t + 16).
__global__ __launch_bounds__(SK_SEL_BLOCK) void snap_sel_write_kernel(SnapArgs a) {
  __shared__ int scan_tmp[SK_SEL_BLOCK / WAVE];
  const int unit = blockIdx.y, n = a.L - a.W;
  const SelState st = a.sel_state[unit];
  int ca = 0, cb = 0;
  const int32_t* cnt = a.sel_counts + size_t(unit) * gridDim.x * 2;
  for (int s = 0; s < int(blockIdx.x); ++s) { ca += cnt[2 * s]; cb += cnt[2 * s + 1]; }
  const float* pv = a.pooled + size_t(unit) * n;
  const int lo = blockIdx.x * SK_SEL_CH + threadIdx.x * SK_SEL_PER;
  uint32_t key[SK_SEL_PER];
  int na = 0, nb = 0;
#pragma unroll
  for (int j = 0; j < SK_SEL_PER; ++j) {
    key[j] = lo + j < n ? ordered_bits(pv[lo + j]) : 0u;
    bool ab, bu;
    sel_classify(key[j], st, ab, bu);
    const bool ok = lo + j < n;
    na += ok && ab;
    nb += ok && bu;
  }
  int total;
  const int packed = block_excl_scan<SK_SEL_BLOCK>((na << 16) | nb, scan_tmp, &total);
  ca += packed >> 16;
  cb += packed & 0xffff;
  int32_t* kept = a.kept + size_t(unit) * a.budget;
#pragma unroll
  for (int j = 0; j < SK_SEL_PER; ++j) {
    if (lo + j < n) {
      bool ab, bu;
      sel_classify(key[j], st, ab, bu);
      if (ab) {
        kept[ca + min(cb, st.r)] = lo + j;
        ++ca;
      } else if (bu) {
        if (cb < st.r) kept[ca + cb] = lo + j;
        ++cb;
      }
    }
  }
}

// grid (row groups, units): copies kept rows of K and V (16-byte words).
__global__ __launch_bounds__(256) void snap_gather_kernel(SnapArgs a, int row_words) {
  const int unit = blockIdx.y;
  const int kept_n = min(a.budget, a.L);
  const int32_t* kept = a.kept + size_t(unit) * a.budget;
  const u32x4* ks = (const u32x4*)a.k + size_t(unit) * a.cap * row_words;
  const u32x4* vs = (const u32x4*)a.v + size_t(unit) * a.cap * row_words;
  u32x4* kd = (u32x4*)a.k_out + size_t(unit) * a.out_cap * row_words;
  u32x4* vd = (u32x4*)a.v_out + size_t(unit) * a.out_cap * row_words;
  const int rows_per_block = 256 / row_words;
  const int i = blockIdx.x * rows_per_block + threadIdx.x / row_words, wd = threadIdx.x % row_words;
  if (threadIdx.x >= rows_per_block * row_words || i >= kept_n) return;
  const int src = kept[i];
  if (src < 0 || src >= a.cap) return;
  kd[size_t(i) * row_words + wd] = ks[size_t(src) * row_words + wd];
  vd[size_t(i) * row_words + wd] = vs[size_t(src) * row_words + wd];
}

// ------------------------------------------------------------------ host
static bool snap_mfma_ok(const se_cache& c, int W) {
  const int R = (c.n_q_heads / c.n_kv_heads) * W;
  return c.dtype == SE_BF16 && (c.d_k == 128 || c.d_k == 64) && R % 64 == 0 && R <= 256;
}

// Compute units of the current device (cached per device).
static int device_cus() {
  static int cus[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (cus[dev] == 0) {
    int n = 0;
    cus[dev] = hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && n > 0 ? n : 256;
  }
  return cus[dev];
}

// Keys per block of the MFMA passes.  Three of their blocks fill a CU, and the
// dispatcher deals blocks to the CUs in a fixed rotation, so the passes take about
// ceil(blocks / resident blocks) rounds of one block's time: the chunk (a multiple of
// 16 keys) minimises rounds x keys per block.  For 32 units of 128K keys on 256 CUs
// it is 912 keys: 4608 blocks, six whole rounds, where 1024 keys made 4096 blocks,
// 5.33 rounds taking the time of 6 (1104 keys, 4.96 rounds, measure the same).
static int snap_chunk_keys(int L, size_t units) {
  const long slots = 3L * device_cus();
  int best = SK_CHUNK_MAX;
  long best_cost = -1;
  for (int ch = SK_CHUNK_MAX; ch >= SK_CHUNK_MIN; ch -= 16) {
    const long blocks = long(units) * ceil_div(L, ch);
    const long cost = (blocks + slots - 1) / slots * ch;
    if (best_cost < 0 || cost < best_cost) { best_cost = cost; best = ch; }
  }
  return best;
}
// chunks of pass A for a given chunk size; the workspace holds partials for the most
// (smallest) chunks any device can be given
static int snap_chunks(int L, int chunk) { return ceil_div(L, chunk); }
static int sel_slices(int n) { return std::max(1, ceil_div(n, SK_SEL_CH)); }

// Workspace: the select's digit histograms first (zero between calls), then its
// state and slice counts, then the score partials, row lse, pooled and votes.
static size_t sel_bytes(size_t units, int n) {
  return units * (SK_SEL_BINS * sizeof(uint32_t) + sizeof(SelState) + size_t(sel_slices(n)) * 2 * sizeof(int32_t));
}

size_t snapkv_ws_bytes(const se_cache& c, int prompt_len, int window) {
  const size_t units = size_t(c.batch) * c.n_kv_heads, R = size_t(c.n_q_heads / c.n_kv_heads) * window;
  const size_t n = size_t(prompt_len - window);
  return sel_bytes(units, int(n)) + units * (size_t(snap_chunks(prompt_len, SK_CHUNK_MIN)) * R * 2 + R + 2 * n) * sizeof(float);
}

// The keep rule and the compaction, from the scores in a.votes: max-pool, top
// (budget - W) of the L - W candidates plus the window, ascending, then the kept
// rows gathered into k_out / v_out.
static se_status snap_keep_compact(const SnapArgs& a, const se_cache& c, hipStream_t s) {
  const size_t units = size_t(a.B) * a.Hkv, n = size_t(a.L - a.W);
  hipLaunchKernelGGL(snap_pool_kernel, dim3(ceil_div(int(n), SK_POOL_T), int(units)), dim3(256), 0, s, a);
  const int kk = std::min(a.budget - a.W, int(n));
  const dim3 sgrid(sel_slices(int(n)), int(units));
  for (int pass = 0; pass < 3; ++pass) {
    hipLaunchKernelGGL(snap_sel_hist_kernel, sgrid, dim3(SK_SEL_BLOCK), 0, s, a, pass);
    hipLaunchKernelGGL(snap_sel_find_kernel, dim3(int(units)), dim3(SK_SEL_BLOCK), 0, s, a, pass, kk);
  }
  hipLaunchKernelGGL(snap_sel_count_kernel, sgrid, dim3(SK_SEL_BLOCK), 0, s, a, kk);
  hipLaunchKernelGGL(snap_sel_write_kernel, sgrid, dim3(SK_SEL_BLOCK), 0, s, a);
  const int esz = c.dtype == SE_F32 ? 4 : 2;
  const int row_words = c.d_k * esz / 16;
  const int rows_per_block = 256 / row_words;
  hipLaunchKernelGGL(snap_gather_kernel, dim3(ceil_div(std::min(a.budget, a.L), rows_per_block), int(units)),
                     dim3(256), 0, s, a, row_words);
  return launch_status();
}

se_status launch_snapkv(const se_cache& c, const void* q_obs, const void* k, const void* v, int prompt_len,
                        int window, int pool_kernel, int budget, float scale, const se_cache& out, void* k_out,
                        void* v_out, int32_t* kept_pos, float* votes, int32_t* out_seq_len, void* ws,
                        hipStream_t s) {
  SnapArgs a{};
  a.q = q_obs; a.k = k; a.v = v; a.k_out = k_out; a.v_out = v_out;
  a.B = c.batch; a.Hq = c.n_q_heads; a.Hkv = c.n_kv_heads; a.G = c.n_q_heads / c.n_kv_heads; a.D = c.d_k;
  a.cap = c.capacity; a.out_cap = out.capacity; a.L = prompt_len; a.W = window; a.R = a.G * window;
  const size_t units = size_t(c.batch) * c.n_kv_heads, n = size_t(prompt_len - window);
  a.pool = pool_kernel; a.budget = budget; a.dtype = c.dtype;
  a.chunk = snap_chunk_keys(prompt_len, units);
  a.nchunks = snap_chunks(prompt_len, a.chunk);
  a.sc2 = scale * SK_LOG2E;
  a.sel_hist = (uint32_t*)ws;
  a.sel_state = (SelState*)(a.sel_hist + units * SK_SEL_BINS);
  a.sel_counts = (int32_t*)(a.sel_state + units);
  float* wsf = (float*)((char*)ws + sel_bytes(units, int(n)));
  a.part = wsf;
  a.lse2 = a.part + units * a.nchunks * a.R * 2;
  a.pooled = a.lse2 + units * a.R;
  a.votes = votes ? votes : a.pooled + units * n;
  a.kept = kept_pos;
  a.out_len = out_seq_len;
  const dim3 vgrid(ceil_div(int(n), 256), int(units));
  if (snap_mfma_ok(c, window)) {
    const int nrb = a.R / 64;
    const dim3 ga(a.nchunks, int(units)), gb(ceil_div(int(n), a.chunk), int(units));
#define SK_LAUNCH(DD, NN)                                                                          \
  do {                                                                                             \
    hipLaunchKernelGGL((snap_mfma_kernel<DD, NN, false>), ga, dim3(256), 0, s, a);                 \
    hipLaunchKernelGGL(snap_lse_merge_kernel, dim3(ceil_div(int(units) * a.R * SK_MERGE_LANES, 256)), dim3(256), 0, s, a); \
    hipLaunchKernelGGL((snap_mfma_kernel<DD, NN, true>), gb, dim3(256), 0, s, a);                  \
  } while (0)
    if (c.d_k == 128) {
      if (nrb == 1) SK_LAUNCH(128, 1); else if (nrb == 2) SK_LAUNCH(128, 2);
      else if (nrb == 3) SK_LAUNCH(128, 3); else SK_LAUNCH(128, 4);
    } else {
      if (nrb == 1) SK_LAUNCH(64, 1); else if (nrb == 2) SK_LAUNCH(64, 2);
      else if (nrb == 3) SK_LAUNCH(64, 3); else SK_LAUNCH(64, 4);
    }
#undef SK_LAUNCH
  } else {
    const size_t lds = size_t(a.R) * a.D * sizeof(float);
    if (lds > 64 * 1024) return SE_ERR_UNSUPPORTED;
    if (c.dtype == SE_F32) {
      hipLaunchKernelGGL(snap_vec_lse_kernel<float>, dim3(a.R, int(units)), dim3(256), a.D * sizeof(float), s, a);
      hipLaunchKernelGGL(snap_vec_vote_kernel<float>, vgrid, dim3(256), lds, s, a);
    } else {
      hipLaunchKernelGGL(snap_vec_lse_kernel<bf16_t>, dim3(a.R, int(units)), dim3(256), a.D * sizeof(float), s, a);
      hipLaunchKernelGGL(snap_vec_vote_kernel<bf16_t>, vgrid, dim3(256), lds, s, a);
    }
  }
  if (hipGetLastError() != hipSuccess) return SE_ERR_HIP;
  return snap_keep_compact(a, c, s);
}

// H2O state at the end of a prefill: scores (two MFMA passes), the keep rule on
// them with no pooling (the heavy best below L - recent, plus the recent window),
// the kept rows gathered into the slot cache, and the slots' positions / scores.
static size_t h2o_prefill_layout(const se_cache& c, int L, int recent, size_t* off) {
  const size_t units = size_t(c.batch) * c.n_kv_heads, G = c.n_q_heads / c.n_kv_heads;
  const size_t n = size_t(L - recent), budget = size_t(L);   // kept rows per unit: at most L
  size_t o = sel_bytes(units, int(n));
  off[0] = o; o += units * n * sizeof(float);                 // pooled
  off[1] = o; o += units * n * sizeof(float);                 // candidate scores (votes)
  off[2] = o; o += (units * budget * sizeof(int32_t) + 15) / 16 * 16;   // kept positions
  off[3] = o; o += (size_t(c.batch) * sizeof(int32_t) + 15) / 16 * 16;  // kept counts
  off[4] = o; o += units * G * size_t(L) * sizeof(float);     // row log2-sum-exp2
  off[5] = o; o += units * size_t(L) * sizeof(float);         // scores of every key
  return o;
}

size_t h2o_prefill_ws_bytes(const se_cache& c, int L, int recent) {
  size_t off[6];
  return h2o_prefill_layout(c, L, recent, off);
}

se_status launch_h2o_prefill(const se_cache& c, const void* q, const void* k, const void* v, int L, int heavy,
                             int recent, float scale, const se_cache& slots, void* k_slots, void* v_slots,
                             int32_t* slot_pos, float* acc, float* scores_out, void* ws, hipStream_t s) {
  size_t off[6];
  h2o_prefill_layout(c, L, recent, off);
  char* w = (char*)ws;
  float* acc0 = scores_out ? scores_out : (float*)(w + off[5]);
  se_status st = launch_h2o_prefill_scores(c, q, k, L, L - recent, scale, (float*)(w + off[4]), acc0,
                                           (float*)(w + off[1]), s);
  if (st != SE_OK) return st;
  SnapArgs a{};
  a.k = k; a.v = v; a.k_out = k_slots; a.v_out = v_slots;
  a.B = c.batch; a.Hq = c.n_q_heads; a.Hkv = c.n_kv_heads; a.G = c.n_q_heads / c.n_kv_heads; a.D = c.d_k;
  a.cap = c.capacity; a.out_cap = slots.capacity; a.L = L; a.W = recent; a.R = 0; a.pool = 1;
  a.budget = std::min(heavy + recent, L); a.nchunks = 0; a.dtype = c.dtype; a.sc2 = 0.f;
  a.sel_hist = (uint32_t*)ws;
  const size_t units = size_t(a.B) * a.Hkv;
  a.sel_state = (SelState*)(a.sel_hist + units * SK_SEL_BINS);
  a.sel_counts = (int32_t*)(a.sel_state + units);
  a.pooled = (float*)(w + off[0]);
  a.votes = (float*)(w + off[1]);
  a.kept = (int32_t*)(w + off[2]);
  a.out_len = (int32_t*)(w + off[3]);
  st = snap_keep_compact(a, c, s);
  if (st != SE_OK) return st;
  return launch_h2o_state(slots, a.kept, a.budget, a.out_len, acc0, L, slot_pos, acc, s);
}

}  // namespace se
