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

// 2^x from v_exp_f32 alone.  Results below 2^-126 come out as zero; exp2f adds
// five VALU operations around the same instruction only to produce those
// subnormal results.  A softmax denominator holds a term >= 2^0 (the running
// maximum's own), so a dropped term is below its rounding; a sum of
// probabilities loses at most 2^-126 per term.
__device__ __forceinline__ float ex2(float x) { return __builtin_amdgcn_exp2f(x); }
// e^x as one multiply and v_exp_f32 (results below 2^-126 come out as zero): the H2O
// score accumulation, in every kernel that computes it, so that the fused decode step
// and the separate calls agree bit for bit
__device__ __forceinline__ float h2o_exp(float x) { return ex2(x * 1.4426950408889634f); }
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
// Wave-wide scans and reductions on DPP lane moves (no LDS round trips): a
// Hillis-Steele scan inside each 16-lane row (row_shr 1, 2, 4, 8), then the
// last lane of row 0 / 1 is broadcast into rows 1, 3 (row_bcast:15) and of
// row 1 into rows 2, 3 (row_bcast:31).  A lane whose DPP source does not exist
// keeps `identity`.
template <class Op>
__device__ __forceinline__ uint32_t wave_incl_scan_dpp(uint32_t v, uint32_t identity, Op op) {
  const int id = int(identity);
  v = op(v, uint32_t(__builtin_amdgcn_update_dpp(id, int(v), 0x111, 0xf, 0xf, false)));   // row_shr:1
  v = op(v, uint32_t(__builtin_amdgcn_update_dpp(id, int(v), 0x112, 0xf, 0xf, false)));   // row_shr:2
  v = op(v, uint32_t(__builtin_amdgcn_update_dpp(id, int(v), 0x114, 0xf, 0xf, false)));   // row_shr:4
  v = op(v, uint32_t(__builtin_amdgcn_update_dpp(id, int(v), 0x118, 0xf, 0xf, false)));   // row_shr:8
  v = op(v, uint32_t(__builtin_amdgcn_update_dpp(id, int(v), 0x142, 0xa, 0xf, false)));   // row_bcast:15
  v = op(v, uint32_t(__builtin_amdgcn_update_dpp(id, int(v), 0x143, 0xc, 0xf, false)));   // row_bcast:31
  return v;
}
// Maximum over each 16-lane row, in every lane of the row, by DPP lane moves:
// quad_perm [1,0,3,2] and [2,3,0,1] give each lane its quad's maximum,
// row_half_mirror (lane i <- 7 - i) joins the two quads of each half row and
// row_mirror (lane i <- 15 - i) the two halves.
__device__ __forceinline__ float row16_max(float v) {
  v = fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0xb1, 0xf, 0xf, false)));
  v = fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x4e, 0xf, 0xf, false)));
  v = fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x141, 0xf, 0xf, false)));
  v = fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x140, 0xf, 0xf, false)));
  return v;
}
// Maximum / sum over the four 16-lane rows of a wave (lanes l, l ^ 16, l ^ 32,
// l ^ 48), in every lane, by the row swaps of gfx950: v_permlane16_swap hands each
// lane the pair {row 2i, row 2i + 1} of its column, v_permlane32_swap the pair of
// half waves, always in that order, so every lane gets the same value (the same
// one as exchanges across 16, then 32, since + and max are commutative).
__device__ __forceinline__ float rows4_max(float v) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto c = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(c[0]), __uint_as_float(c[1]));
}
__device__ __forceinline__ float rows4_sum(float v) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const auto c = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(c[0]) + __uint_as_float(c[1]);
}
// Inclusive scan inside each 16-lane row only (lane 15 of a row ends with the row's total).
template <class Op>
__device__ __forceinline__ uint32_t row_incl_scan_dpp(uint32_t v, uint32_t identity, Op op) {
  const int id = int(identity);
  v = op(v, uint32_t(__builtin_amdgcn_update_dpp(id, int(v), 0x111, 0xf, 0xf, false)));   // row_shr:1
  v = op(v, uint32_t(__builtin_amdgcn_update_dpp(id, int(v), 0x112, 0xf, 0xf, false)));   // row_shr:2
  v = op(v, uint32_t(__builtin_amdgcn_update_dpp(id, int(v), 0x114, 0xf, 0xf, false)));   // row_shr:4
  v = op(v, uint32_t(__builtin_amdgcn_update_dpp(id, int(v), 0x118, 0xf, 0xf, false)));   // row_shr:8
  return v;
}
// Value of the last lane (the wave-wide reduction) as a wave-uniform value.
__device__ __forceinline__ uint32_t wave_last(uint32_t v) { return uint32_t(__builtin_amdgcn_readlane(int(v), 63)); }

__device__ __forceinline__ uint32_t wave_or(uint32_t v) {
  return wave_last(wave_incl_scan_dpp(v, 0u, [](uint32_t a, uint32_t b) { return a | b; }));
}
__device__ __forceinline__ uint32_t wave_and(uint32_t v) {
  return wave_last(wave_incl_scan_dpp(v, ~0u, [](uint32_t a, uint32_t b) { return a & b; }));
}
__device__ __forceinline__ float wave_max(float v) {
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, WAVE));
  return v;
}
__device__ __forceinline__ float wave_sum(float v) {
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, WAVE);
  return v;
}
__device__ __forceinline__ int wave_sum_i(int v) {
  return int(wave_last(wave_incl_scan_dpp(uint32_t(v), 0u, [](uint32_t a, uint32_t b) { return a + b; })));
}
// Inclusive prefix sum across the wave (every lane of the wave active).
__device__ __forceinline__ int wave_incl_scan(int v) {
  return int(wave_incl_scan_dpp(uint32_t(v), 0u, [](uint32_t a, uint32_t b) { return a + b; }));
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

// ------------------------------------------------------------------ cross-block completion
// A launch whose blocks each finish a share of some unit's work lets the block
// that finishes last complete it (a top-k over all page scores, a merge of
// split partials) inside the same launch.  The blocks of one unit run on
// different XCDs, whose L2 caches are not coherent with each other, and a
// device-scope fence would write back or invalidate a whole L2, stalling every
// block streaming through that XCD.  So the shared data is written and read
// only with relaxed device-scope atomic accesses (sc1 stores that write
// through to the coherence point, sc1 loads that read from it); a block waits
// for its stores to complete before it takes its ticket, and the last block
// issues its loads only after its ticket shows every share done.
__device__ __forceinline__ void st_dev(float* p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float ld_dev(const float* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// Two consecutive floats at an 8-byte aligned address, as one access.
__device__ __forceinline__ void st_dev2(float* p, float x, float y) {
  const uint64_t v = (uint64_t(__float_as_uint(y)) << 32) | __float_as_uint(x);
  __hip_atomic_store(reinterpret_cast<uint64_t*>(p), v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float2 ld_dev2(const float* p) {
  const uint64_t v = __hip_atomic_load(reinterpret_cast<const uint64_t*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  return make_float2(__uint_as_float(uint32_t(v)), __uint_as_float(uint32_t(v >> 32)));
}
// Takes this block's ticket on `ctr`; true in the block that takes ticket nblocks - 1.
__device__ __forceinline__ bool block_ticket_last(int* ctr, int nblocks) {
  __shared__ int s_last;
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_waitcnt(0);     // this thread's stores have completed
  __syncthreads();
  if (threadIdx.x == 0)
    s_last = __hip_atomic_fetch_add(ctr, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == nblocks - 1;
  __syncthreads();
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  return s_last != 0;
}
// The last block returns the counter to zero for the next launch.
__device__ __forceinline__ void ticket_reset(int* ctr) {
  __hip_atomic_store(ctr, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
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


// Register-resident variant for n <= BLOCK * E.  Wave w owns candidates
// [64 E w, 64 E (w + 1)); its lane l holds 64 E w + 64 j + l for j < E, so
// every load is coalesced.  Keys are 32-bit ordered scores; slots past n hold
// key 0, which is below every real key (ordered_bits of a non-NaN float is
// never 0), so they never enter the kept set and need no masks.  Radix select
// on the score bits: the bits every candidate shares are skipped, then 8-bit
// digits are counted in LDS histograms private to each wave (zeroed by that wave),
// COPIES of them per wave with lane l counting into copy l % COPIES: scores cluster
// in few digits, and LDS atomics to one address from the lanes of an instruction
// are serialized, so copies divide that serialization, while each copy adds to the
// clearing and to the scan (two copies measured best in the in-launch selections of
// the decode attention; four and eight were slower).  Wave 0 alone scans the digit
// counts (DPP) and posts the crossing digit, so a digit pass costs two block
// barriers.  The search stops when one digit bucket holds exactly the keys still
// to choose, or when all 32 bits are resolved.
// The kept set is every key above the resolved prefix plus the first `r` keys
// of the prefix's bucket in index order (the lower-index tie rule); per-wave
// counts give each wave its output offset and ballot prefix counts place each
// kept candidate, so the view comes out in ascending index order.
template <int NWAVES, int COPIES = 1>
struct TopkRegSharedN {
  static constexpr int copies = COPIES;
  uint32_t hist[NWAVES][COPIES][256];   // per wave, lane l counting into copy l % COPIES
  uint32_t red_or[NWAVES], red_and[NWAVES];
  int cnt_a[NWAVES], cnt_b[NWAVES];
  int digit, rem, cnt;
};
using TopkRegShared = TopkRegSharedN<16>;   // blocks of up to 1024 threads

__device__ __forceinline__ int lanes_below(uint64_t m) {
  return int(__builtin_amdgcn_mbcnt_hi(uint32_t(m >> 32), __builtin_amdgcn_mbcnt_lo(uint32_t(m), 0u)));
}

struct TopkNoHook {
  __device__ void operator()() const {}
};

// The candidate this thread's key j stands for in block_topk_reg / block_topk_keys.
template <int BLOCK, int E>
__device__ __forceinline__ int topk_reg_index(int j) {
  return (int(threadIdx.x) / WAVE) * WAVE * E + (int(threadIdx.x) & (WAVE - 1)) + j * WAVE;
}

template <int BLOCK, int E, class SH>
__device__ int block_topk_keys(uint32_t (&key)[E], int n, int k, int32_t* out, SH& sh);

// after_loads() runs once every key load has been issued (its own memory operations
// then overlap those loads' return)
template <int BLOCK, int E, class LoadFn, class SH, class AfterLoads = TopkNoHook>
__device__ int block_topk_reg(LoadFn load, int n, int k, int32_t* out, SH& sh,
                              AfterLoads after_loads = AfterLoads{}) {
  uint32_t key[E];
  // unconditional loads at a clamped index (element 0 always exists), masked after:
  // all E loads go out together instead of one guarded round trip each
#pragma unroll
  for (int j = 0; j < E; ++j) {
    const int i = topk_reg_index<BLOCK, E>(j);
    const uint32_t v = ordered_bits(load(max(min(i, n - 1), 0)));
    key[j] = i < n ? v : 0u;
  }
  after_loads();
  return block_topk_keys<BLOCK, E, SH>(key, n, k, out, sh);
}

// The selection itself, on keys already in registers: key[j] is ordered_bits of the
// score of candidate topk_reg_index(j), or 0 where that index is not a candidate.
template <int BLOCK, int E, class SH>
__device__ int block_topk_keys(uint32_t (&key)[E], int n, int k, int32_t* out, SH& sh) {
  static_assert(BLOCK >= 64 && BLOCK <= 1024 && BLOCK % WAVE == 0, "block size");
  constexpr int NW = BLOCK / WAVE;
  static_assert(sizeof(sh.red_or) / sizeof(sh.red_or[0]) >= NW, "shared state for every wave");
  const int tid = threadIdx.x, lane = tid & (WAVE - 1), w = tid / WAVE;
  const int kk = k < n ? k : n;
  const int base = w * WAVE * E + lane;
  uint32_t mask = 0u, prefix = 0u;   // resolved top bits and their value
  int r = kk;                        // keys still to take from the bucket (key & mask) == prefix
  if (kk > 0 && kk < n) {
    uint32_t kor = 0u, kand = ~0u;
#pragma unroll
    for (int j = 0; j < E; ++j) {
      kor |= key[j];
      kand &= key[j] | (key[j] == 0u ? ~0u : 0u);   // padding does not clear common bits
    }
    kor = wave_or(kor);
    kand = wave_and(kand);
    if (lane == 0) { sh.red_or[w] = kor; sh.red_and[w] = kand; }
    __syncthreads();
    kor = 0u; kand = ~0u;
#pragma unroll
    for (int i = 0; i < NW; ++i) { kor |= sh.red_or[i]; kand &= sh.red_and[i]; }
    const uint32_t diff = kor ^ kand;
    if (diff == 0u) {
      mask = ~0u;          // every key equal: the first kk by index
      prefix = kand;
    } else {
      const int top = 31 - __clz(diff);
      mask = top == 31 ? 0u : (~0u << (top + 1));
      prefix = kand & mask;
      constexpr int NC = SH::copies;
      uint32_t* hist = sh.hist[w][lane % NC];
      for (int hb = top; hb >= 0; hb -= 8) {
        const int shift = hb >= 7 ? hb - 7 : 0;
        const uint32_t dmask = (1u << (hb - shift + 1)) - 1u;
#pragma unroll
        for (int c = 0; c < NC; ++c)   // in LDS order before this wave's atomics
          reinterpret_cast<uint4*>(sh.hist[w][c])[lane] = make_uint4(0u, 0u, 0u, 0u);
#pragma unroll
        for (int j = 0; j < E; ++j)
          if ((key[j] & mask) == prefix) atomicAdd(&hist[(key[j] >> shift) & dmask], 1u);
        __syncthreads();
        if (w == 0) {
          // lane l owns digits 255 - 4l .. 252 - 4l (descending); an inclusive scan over
          // lanes counts the keys whose digit is >= the lane's lowest
          int c0 = 0, c1 = 0, c2 = 0, c3 = 0;
#pragma unroll
          for (int i = 0; i < NW; ++i)
#pragma unroll
            for (int c = 0; c < NC; ++c) {
              const uint4 h4 = reinterpret_cast<const uint4*>(sh.hist[i][c])[63 - lane];
              c0 += int(h4.w); c1 += int(h4.z); c2 += int(h4.y); c3 += int(h4.x);
            }
          const int own = c0 + c1 + c2 + c3;
          const int incl = wave_incl_scan(own);
          int above = incl - own;
          if (above < r && r <= incl) {
            const int cs[4] = {c0, c1, c2, c3};
#pragma unroll
            for (int j = 0; j < 4; ++j) {
              if (above + cs[j] >= r) {
                sh.digit = 255 - 4 * lane - j;
                sh.rem = r - above;
                sh.cnt = cs[j];
                break;
              }
              above += cs[j];
            }
          }
        }
        __syncthreads();
        const int fd = sh.digit, frem = sh.rem, fcnt = sh.cnt;
        prefix |= uint32_t(fd) << shift;
        mask |= dmask << shift;
        r = frem;
        if (fcnt == frem) break;   // the whole bucket is kept
      }
    }
  }
  // compaction in index order: above = (key & mask) > prefix, bucket = (key & mask) == prefix (real keys only)
  int na = 0, nb = 0;
#pragma unroll
  for (int j = 0; j < E; ++j) {
    const uint32_t km = key[j] & mask;
    na += km > prefix;
    nb += km == prefix && key[j] != 0u;
  }
  na = wave_sum_i(na);
  nb = wave_sum_i(nb);
  if (lane == 0) { sh.cnt_a[w] = na; sh.cnt_b[w] = nb; }
  __syncthreads();
  int ca = 0, cb = 0;
  for (int i = 0; i < w; ++i) { ca += sh.cnt_a[i]; cb += sh.cnt_b[i]; }
#pragma unroll
  for (int j = 0; j < E; ++j) {
    const uint32_t km = key[j] & mask;
    const bool is_a = km > prefix;
    const bool is_b = km == prefix && key[j] != 0u;
    const uint64_t ma = __ballot(is_a), mb = __ballot(is_b);
    const int pa = ca + lanes_below(ma), pb = cb + lanes_below(mb);
    if (is_a) out[pa + min(pb, r)] = base + j * WAVE;
    else if (is_b && pb < r) out[pa + pb] = base + j * WAVE;
    ca += __popcll(ma);
    cb += __popcll(mb);
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
se_status launch_kv_append_meta(const se_cache& c, void* k, void* v, const void* k_new, const void* v_new,
                                const int32_t* slot, int32_t* seq_len, void* kmin, void* kmax, int page_size,
                                hipStream_t s);
size_t quest_ws_bytes(const se_cache& c, int page_size, int top_pages);
size_t quest_append_ws_bytes(const se_cache& c, int page_size);
size_t quest_step_ws_bytes(const se_cache& c, int page_size, int top_pages);
size_t h2o_step_ws_bytes(const se_cache& c);
se_status launch_h2o_step(const se_cache& c, const void* q, void* k, void* v, const void* k_new, const void* v_new,
                          const int32_t* slot_in, int32_t* seq_len, int32_t* slot_pos, float* acc, int cur_pos,
                          int heavy, int recent, float scale, float* out, float* lse, int32_t* evict_out, void* ws,
                          hipStream_t s);
se_status launch_quest_append_scores(const se_cache& c, const void* q, void* k, void* v, const void* k_new,
                                     const void* v_new, const int32_t* seq_len, void* kmin, void* kmax, int page_size,
                                     float* page_score, void* ws, float** score_out, hipStream_t s);
se_status launch_quest_step(const se_cache& c, const void* q, void* k, void* v, const void* k_new,
                            const void* v_new, int32_t* seq_len, void* kmin, void* kmax, int page_size,
                            int top_pages, float scale, float* out, float* lse, int32_t* view_idx,
                            int32_t* view_len, float* page_score, void* ws, hipStream_t s);
se_status launch_quest_fp8_append_scores(const se_cache& c, const void* q, void* kq, void* vq, void* ks, void* vs,
                                         const void* k_new, const void* v_new, const int32_t* seq_len, void* kmin,
                                         void* kmax, int page_size, float* page_score, void* ws, float** score_out,
                                         hipStream_t s);
se_status launch_quest_step_fp8(const se_cache& c, const void* q, void* kq, void* vq, uint8_t* ks, uint8_t* vs,
                                const void* k_new, const void* v_new, int32_t* seq_len, void* kmin, void* kmax,
                                int page_size, int top_pages, float scale, float* out, float* lse, int32_t* view_idx,
                                int32_t* view_len, float* page_score, void* ws, hipStream_t s);
se_status launch_streaming_view(const se_cache& c, const int32_t* seq_len, int sink, int recent,
                                int32_t* view_idx, int32_t* view_len, int view_cap, int pending, hipStream_t s);
void pyramid_budgets(int n, int avg, int bmin, int32_t* out);
se_status launch_h2o_prefill_scores(const se_cache& c, const void* q, const void* k, int L, int n_cand, float scale,
                                    float* lse2, float* acc0, float* votes, hipStream_t s);
se_status launch_h2o_state(const se_cache& c_slots, const int32_t* kept, int kept_stride, const int32_t* kept_len,
                           const float* acc0, int L, int32_t* slot_pos, float* acc, hipStream_t s);
size_t h2o_prefill_ws_bytes(const se_cache& c, int L, int recent);
se_status launch_h2o_prefill(const se_cache& c, const void* q, const void* k, const void* v, int L, int heavy,
                             int recent, float scale, const se_cache& slots, void* k_slots, void* v_slots,
                             int32_t* slot_pos, float* acc, float* scores_out, void* ws, hipStream_t s);
void chain_match(const int32_t* tokens, int n_tokens, const int32_t* const* prefixes, const int32_t* lens,
                 int n_prefixes, int32_t* session, int32_t* matched);
se_status launch_chain_remap(const se_cache& c, const int32_t* map_in, int cap_in, const int32_t* kept,
                             int kept_stride, const int32_t* kept_len, int32_t* map_out, hipStream_t s);
se_status launch_chain_append(const se_cache& c, int32_t* pos_map, const int32_t* seq_len, const int32_t* logical_len,
                              int n_new, hipStream_t s);
se_status launch_quest_append(const se_cache& c, const void* q, void* k, void* v, const void* k_new,
                              const void* v_new, int32_t* seq_len, void* kmin, void* kmax, int page_size,
                              int top_pages, int32_t* view_idx, int32_t* view_len, float* page_score, void* ws,
                              hipStream_t s);
se_status launch_quest(const se_cache& c, const void* q, const void* kmin, const void* kmax,
                       const int32_t* seq_len, int page_size, int top_pages, int32_t* view_idx,
                       int32_t* view_len, float* page_score, void* ws, hipStream_t s);
int attn_auto_splits(const se_cache& c, int slots);
size_t attn_counter_bytes(const se_cache& c);   // leading ticket-counter bytes of an attention workspace
size_t attn_ws_bytes(const se_cache& c, int slots, int num_splits);
// k_scale / v_scale non-null: K / V hold FP8 rows with one scale byte per row.
size_t attn_append_ws_bytes(const se_cache& c, int slots, int num_splits);
se_status launch_append_attn(const se_cache& c, const void* q, void* k, void* v, const void* k_new,
                             const void* v_new, const int32_t* slot, int32_t* seq_len, const int32_t* view_idx,
                             const int32_t* view_len, int view_cap, int granularity, float scale, float* out,
                             float* lse, float* logits, int logit_cap, int num_splits, void* ws, hipStream_t s);
se_status launch_attn(const se_cache& c, const void* q, const void* k, const void* v,
                      const int32_t* seq_len, const int32_t* view_idx, const int32_t* view_len,
                      int view_cap, int granularity, float scale, float* out, float* lse,
                      float* logits, int logit_cap, int num_splits, void* ws, hipStream_t s,
                      const uint8_t* k_scale = nullptr, const uint8_t* v_scale = nullptr);
se_status launch_fp8_quantize(const se_cache& c, const void* k, const void* v, const int32_t* seq_len, void* kq,
                              void* vq, void* ks, void* vs, void* kmin, void* kmax, int page_size, hipStream_t s);
se_status launch_fp8_append(const se_cache& c, void* kq, void* vq, void* ks, void* vs, const void* k_new,
                            const void* v_new, int32_t* seq_len, void* kmin, void* kmax, int page_size, hipStream_t s);
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
