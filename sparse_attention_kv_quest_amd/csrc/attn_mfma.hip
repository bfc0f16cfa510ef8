// bf16 GQA split-K decode attention on MFMA (gfx950, v_mfma_f32_16x16x32_bf16).
//
// The G query heads of a KV head share every K/V row they read, so both
// products of decode attention are small dense contractions:
//   S^T[token][head] = K[token][:] . Q[head][:]      (A = K rows, B = Q^T)
//   O^T[dim][head]  += V^T[dim][token] . P^T[token][head]
// Heads are padded to 16 columns.  K rows go straight from HBM into the MFMA
// A-operand registers (per load instruction, 16 rows x 64 contiguous bytes);
// V rows are transposed through a wave-private LDS tile so that every lane
// holds eight tokens of one dimension.  Softmax runs in fp32; P enters the
// second product as a bf16 hi + lo pair, so the rounding of P costs ~2^-17
// relative.
//
// Work split: a block of 4 waves owns a contiguous chunk of one unit's view
// slots (split-K).  Each wave walks every fourth 32-slot tile of the chunk
// with the next tile's K/V loads in flight while it computes the current one
// (registers double-buffered: two waves per SIMD for d 128, or one wave per
// SIMD with two tiles in flight), so HBM sees a continuous stream.  The view
// entries of the chunk are cached in LDS first, so a token lookup never waits
// on the loads in flight.  The running max of a head is
// only moved (and the output rescaled) when a tile's max exceeds it by more
// than 2^8, which keeps the accumulators untouched on almost every tile; the
// shift cancels in the final normalisation.  The four waves merge their
// (max, sum, output) in LDS and the block writes one partial; the block that
// finishes a unit's last split merges the splits, so a call is one launch.
#include <type_traits>

#include "attn_common.hpp"
#include "mfma_util.hpp"

namespace se {

constexpr int MF_TS = 32;         // view slots per wave tile
constexpr int MF_WAVES = 4;
constexpr int MF_VCACHE = 2048;   // view entries cached in LDS per block
constexpr float MF_RESCALE_MARGIN = 8.f;   // log2 units

template <int D>
struct MfTile {
  u32x4 k0[D / 32], k1[D / 32];   // K rows of slots base + c16 and base + 16 + c16
  u32x4 v[D / 64][4];             // V rows of slots base + 4 (lane & 7) + r, 8-dim chunks
  int tk0, tk1;
};

// FP8 rows as loaded: 16 K bytes of rows tk0 / tk1 per 64-byte span, lane group g
// holding bytes 64 j + 16 g .. + 15 (so each load reads 64 contiguous bytes of 16
// rows; k-step c takes the 8 bytes from 64 (c / 2) + 16 g + 8 (c % 2) on, and q is
// staged in the same order), 8 V bytes per row and pass (where d is a multiple of
// 128 a pass pair's 16 bytes are contiguous: dims 16 (lane >> 3) + 128 k on; else
// the bf16 layout's dims), and every row's scale byte.
template <int D>
struct MfTileF8 {
  u32x4 k0[D / 64], k1[D / 64];
  uint2 v[D / 64][4];
  uint32_t ks0, ks1, vs[4];
  int tk0, tk1;
};

template <int D, bool F8>
using MfRaw = std::conditional_t<F8, MfTileF8<D>, MfTile<D>>;

struct MfCtx {
  const uint16_t* ku;
  const uint16_t* vu;
  const uint8_t* ksc;    // FP8: scale bytes of the unit's rows
  const uint8_t* vsc;
  const int32_t* vglob;  // view entries in global memory (used when they do not fit the LDS cache)
  const uint16_t* knew;  // fused append: the unit's new K / V rows, read in place of cache slot tgt
  const uint16_t* vnew;
  int e0, len, s1, gshift;
  int tgt;               // fused append: the slot receiving the new row (-2: none)
  bool identity;
};

__shared__ int32_t mf_vcache[MF_VCACHE];

// Cache slot read by view slot s, or -1 (power-of-two granularity 1 << gshift).
// VC: the view entries come from the LDS cache.
template <bool VC>
__device__ __forceinline__ int mf_token(const MfCtx& x, int s) {
  int t;
  if (x.identity) {
    t = s;
  } else {
    const int e = s >> x.gshift;
    int page;
    if (VC) {   // read unconditionally (clamped index): no branch, no wait per lookup
      const int pv = mf_vcache[min(max(e - x.e0, 0), MF_VCACHE - 1)];
      page = s < x.s1 ? pv : -1;
    } else {
      page = s < x.s1 ? x.vglob[e] : -1;
    }
    t = page < 0 ? -1 : (page << x.gshift) + (s & ((1 << x.gshift) - 1));
  }
  return (s < x.s1 && t >= 0 && t < x.len) ? t : -1;
}

template <int D, bool VC, bool APP = false>
__device__ __forceinline__ void mf_load(const MfCtx& x, int base, int lane, MfTile<D>& T) {
  constexpr int NKS = D / 32, VPASS = D / 64;
  const int g = lane >> 4, c16 = lane & 15, qa = lane & 7;
  T.tk0 = mf_token<VC>(x, base + c16);
  T.tk1 = mf_token<VC>(x, base + 16 + c16);
  int vtok[4];
  const int sq = base + 4 * qa;
  if (x.identity || x.gshift >= 2) {   // a 4-aligned slot quad stays inside one view entry
    const int t0 = mf_token<VC>(x, sq);
#pragma unroll
    for (int r = 0; r < 4; ++r) vtok[r] = (t0 >= 0 && sq + r < x.s1 && t0 + r < x.len) ? t0 + r : -1;
  } else {
#pragma unroll
    for (int r = 0; r < 4; ++r) vtok[r] = mf_token<VC>(x, sq + r);
  }
  // Loads are unconditional: a slot without a token reads the unit's row 0, which is
  // finite data; its K is masked through the logits and its weight p is 0.  Keeping
  // the loads unconditional keeps the compiler's wait counters exact across the
  // prefetch.  Offsets stay 32-bit within the unit.
  const uint32_t r0 = uint32_t(max(T.tk0, 0)) * D + 8 * g, r1 = uint32_t(max(T.tk1, 0)) * D + 8 * g;
  if constexpr (APP) {   // the slot receiving the new row reads it from k_new / v_new
    const uint16_t* p0 = T.tk0 == x.tgt ? x.knew + 8 * g : x.ku + r0;
    const uint16_t* p1 = T.tk1 == x.tgt ? x.knew + 8 * g : x.ku + r1;
#pragma unroll
    for (int c = 0; c < NKS; ++c) {
      T.k0[c] = ld16(p0 + 32 * c);
      T.k1[c] = ld16(p1 + 32 * c);
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const uint16_t* pv = vtok[r] == x.tgt ? x.vnew + 8 * (lane >> 3) : x.vu + uint32_t(max(vtok[r], 0)) * D + 8 * (lane >> 3);
#pragma unroll
      for (int p = 0; p < VPASS; ++p) T.v[p][r] = ld16(pv + 64 * p);
    }
  } else {
#pragma unroll
    for (int c = 0; c < NKS; ++c) {
      T.k0[c] = ld16(x.ku + r0 + 32 * c);
      T.k1[c] = ld16(x.ku + r1 + 32 * c);
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const uint32_t rv = uint32_t(max(vtok[r], 0)) * D + 8 * (lane >> 3);
#pragma unroll
      for (int p = 0; p < VPASS; ++p) T.v[p][r] = ld16(x.vu + rv + 64 * p);
    }
  }
}

// Scale 2^(s - 127) of a scale byte, clamped to the normal float range.
__device__ __forceinline__ float mf_scale(uint32_t sb) { return __uint_as_float(min(max(sb, 1u), 254u) << 23); }

// Four bf16 pairs (8 values) of the 8 FP8 codes in w0, w1, each times `sc` (exact).
__device__ __forceinline__ u32x4 mf_cvt8(uint32_t w0, uint32_t w1, float sc) {
  typedef __bf16 bf2 __attribute__((ext_vector_type(2)));
  const bf2 a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w0, sc, false);
  const bf2 b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w0, sc, true);
  const bf2 c = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w1, sc, false);
  const bf2 d = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w1, sc, true);
  return u32x4{__builtin_bit_cast(uint32_t, a), __builtin_bit_cast(uint32_t, b), __builtin_bit_cast(uint32_t, c),
               __builtin_bit_cast(uint32_t, d)};
}

template <int D, bool VC>
__device__ __forceinline__ void mf_load_f8(const MfCtx& x, int base, int lane, MfTileF8<D>& T) {
  constexpr int VPASS = D / 64;
  const int g = lane >> 4, c16 = lane & 15, qa = lane & 7;
  T.tk0 = mf_token<VC>(x, base + c16);
  T.tk1 = mf_token<VC>(x, base + 16 + c16);
  int vtok[4];
  const int sq = base + 4 * qa;
  if (x.identity || x.gshift >= 2) {
    const int t0 = mf_token<VC>(x, sq);
#pragma unroll
    for (int r = 0; r < 4; ++r) vtok[r] = (t0 >= 0 && sq + r < x.s1 && t0 + r < x.len) ? t0 + r : -1;
  } else {
#pragma unroll
    for (int r = 0; r < 4; ++r) vtok[r] = mf_token<VC>(x, sq + r);
  }
  // unconditional loads, as in the bf16 tile (slots without a token read row 0)
  const uint8_t* ku = reinterpret_cast<const uint8_t*>(x.ku);
  const uint8_t* vu = reinterpret_cast<const uint8_t*>(x.vu);
  const uint32_t t0 = uint32_t(max(T.tk0, 0)), t1 = uint32_t(max(T.tk1, 0));
#pragma unroll
  for (int j = 0; j < D / 64; ++j) {
    T.k0[j] = ld16(ku + t0 * D + 16 * g + 64 * j);
    T.k1[j] = ld16(ku + t1 * D + 16 * g + 64 * j);
  }
  T.ks0 = x.ksc[t0];
  T.ks1 = x.ksc[t1];
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const uint32_t tv = uint32_t(max(vtok[r], 0));
    if constexpr (VPASS % 2 == 0) {
      // one 16-byte load per pass pair: dims 16 (lane >> 3) + 128 k .. + 15, so each
      // load of the wave covers eight whole 128-byte rows
#pragma unroll
      for (int k = 0; k < VPASS / 2; ++k) {
        const u32x4 w = ld16(vu + tv * D + 16 * (lane >> 3) + 128 * k);
        T.v[2 * k][r] = uint2{w[0], w[1]};
        T.v[2 * k + 1][r] = uint2{w[2], w[3]};
      }
    } else {
#pragma unroll
      for (int p = 0; p < VPASS; ++p) T.v[p][r] = *reinterpret_cast<const uint2*>(vu + tv * D + 8 * (lane >> 3) + 64 * p);
    }
    T.vs[r] = x.vsc[tv];
  }
}

// The MFMA operands of a tile: bf16 tiles as loaded; FP8 tiles converted at their use
// (K per k-step, V per pass), so no converted copy of a whole tile is held.
template <int D>
__device__ __forceinline__ u32x4 mf_kop(const MfTile<D>& T, int half, int c) { return half ? T.k1[c] : T.k0[c]; }
template <int D>
__device__ __forceinline__ u32x4 mf_kop(const MfTileF8<D>& T, int half, int c) {
  const int j = c / 2, w = 2 * (c % 2);   // k-step c: bytes 64 j + 16 g + 4 w .. + 7 of the row
  const u32x4& src = half ? T.k1[j] : T.k0[j];
  return mf_cvt8(src[w], src[w + 1], mf_scale(half ? T.ks1 : T.ks0));
}
template <int D>
__device__ __forceinline__ u32x4 mf_vop(const MfTile<D>& T, int pp, int r) { return T.v[pp][r]; }
// The 8-dim V chunk a lane holds in pass pp (its dims are 8 ch .. 8 ch + 7).
template <int D>
__device__ __forceinline__ int mf_vch(const MfTile<D>&, int lane, int pp) { return (lane >> 3) + 8 * pp; }
template <int D>
__device__ __forceinline__ int mf_vch(const MfTileF8<D>&, int lane, int pp) {
  if constexpr ((D / 64) % 2 == 0) return 2 * (lane >> 3) + 16 * (pp >> 1) + (pp & 1);
  else return (lane >> 3) + 8 * pp;
}
template <int D>
__device__ __forceinline__ u32x4 mf_vop(const MfTileF8<D>& T, int pp, int r) {
  return mf_cvt8(T.v[pp][r].x, T.v[pp][r].y, mf_scale(T.vs[r]));
}

template <int D>
struct MfState {
  f32x4 o[D / 16];
  float m2, lsum;
};

template <int D, class TT>
__device__ __forceinline__ void mf_compute(const AttnArgs& a, const MfCtx& x, int base, int lane, const u32x4* qv,
                                           float sc2, float* lg_base, float* lgs, uint16_t* vt, const TT& T,
                                           MfState<D>& st) {
  constexpr int NKS = D / 32, NDB = D / 16, VPASS = D / 64, PITCH = MF_TS + 4;
  const int g = lane >> 4, c16 = lane & 15, qa = lane & 7;
  // ---- S^T = K Q^T for the two 16-slot blocks
  f32x4 sa = {0.f, 0.f, 0.f, 0.f}, sb = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int c = 0; c < NKS; ++c) {
    sa = mfma_bf16_16x16x32(mf_kop<D>(T, 0, c), qv[c], sa);
    sb = mfma_bf16_16x16x32(mf_kop<D>(T, 1, c), qv[c], sb);
  }
  const uint64_t va = __ballot(T.tk0 >= 0), vb = __ballot(T.tk1 >= 0);
  float sv[8];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const bool oka = (va >> (4 * g + i)) & 1, okb = (vb >> (4 * g + i)) & 1;
    sv[i] = oka ? sa[i] * sc2 : -INFINITY;
    sv[4 + i] = okb ? sb[i] * sc2 : -INFINITY;
  }
  if (lg_base != nullptr) {
    // the tile's [head][slot] logits go through the wave's LDS staging rows and are
    // stored after P.V (fewer registers live there), each head's 32 slots as one
    // contiguous run
    constexpr int LP = MF_TS + 4;
    float* lt = lgs;
    f32x4 la, lb;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      la[i] = ((va >> (4 * g + i)) & 1) ? sa[i] * a.scale : -INFINITY;
      lb[i] = ((vb >> (4 * g + i)) & 1) ? sb[i] * a.scale : -INFINITY;
    }
    *reinterpret_cast<f32x4*>(lt + c16 * LP + 4 * g) = la;
    *reinterpret_cast<f32x4*>(lt + c16 * LP + 16 + 4 * g) = lb;
  }
  // ---- online softmax; head c16 lives in lanes c16, c16+16, c16+32, c16+48
  float tmax = sv[0];
#pragma unroll
  for (int i = 1; i < 8; ++i) tmax = fmaxf(tmax, sv[i]);
  tmax = rows4_max(tmax);
  // move the running max only when this tile exceeds it by more than the margin
  const bool grow = tmax > st.m2 + MF_RESCALE_MARGIN;
  if (__ballot(grow) != 0) {
    const float mnew = grow ? tmax : st.m2;
    const float alpha = (grow && st.m2 != -INFINITY) ? ex2(st.m2 - mnew) : 1.f;
    st.lsum *= alpha;
#pragma unroll
    for (int i = 0; i < NDB; ++i) st.o[i] *= alpha;
    st.m2 = mnew;
  }
  // while no valid slot has been seen the max stays -inf and every logit is -inf
  const float mref = st.m2 == -INFINITY ? 0.f : st.m2;
  float p[8];
  float psum = 0.f;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    p[i] = ex2(sv[i] - mref);   // 0 for masked slots; at most 2^8 otherwise
    psum += p[i];
  }
  st.lsum += psum;
  // P as the B operand, split into bf16 hi + lo
  u32x4 ph, pl;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const uint32_t h = pack_bf16(p[2 * j], p[2 * j + 1]);
    ph[j] = h;
    pl[j] = pack_bf16(p[2 * j] - bf16x2_lo_f32(h), p[2 * j + 1] - bf16x2_hi_f32(h));
  }
  // ---- V quads -> transposed LDS tile: row = dim, 32 tokens per row
#pragma unroll
  for (int pp = 0; pp < VPASS; ++pp) {
    const int ch = mf_vch<D>(T, lane, pp);
    u32x4 vv[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) vv[r] = mf_vop<D>(T, pp, r);
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      const uint32_t w0 = vv[0][m], w1 = vv[1][m], w2 = vv[2][m], w3 = vv[3][m];
      uint2 lo, hi;
      lo.x = lo16_pair(w0, w1);
      lo.y = lo16_pair(w2, w3);
      hi.x = hi16_pair(w0, w1);
      hi.y = hi16_pair(w2, w3);
      *reinterpret_cast<uint2*>(vt + (8 * ch + 2 * m) * PITCH + 4 * qa) = lo;
      *reinterpret_cast<uint2*>(vt + (8 * ch + 2 * m + 1) * PITCH + 4 * qa) = hi;
    }
  }
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  // ---- O^T += V^T P^T
#pragma unroll
  for (int db = 0; db < NDB; ++db) {
    const uint16_t* row = vt + (16 * db + c16) * PITCH;
    const uint2 x0 = *reinterpret_cast<const uint2*>(row + 4 * g);
    const uint2 x1 = *reinterpret_cast<const uint2*>(row + 16 + 4 * g);
    const u32x4 av = {x0.x, x0.y, x1.x, x1.y};
    st.o[db] = mfma_bf16_16x16x32(av, ph, st.o[db]);
    st.o[db] = mfma_bf16_16x16x32(av, pl, st.o[db]);
  }
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  if (lg_base != nullptr) {   // this tile's logits, staged above (the barriers above ordered them)
    constexpr int LP = MF_TS + 4;
    const float* lt = lgs;
    const int sl = base + (lane & 31);
    const bool sok = sl < x.s1 && sl < a.logit_cap;
    // offsets within the group's rows (G * logit_cap < 2^31): one per-lane term, the
    // head pair's part uniform, so no per-head pointer stays live across tiles
    const uint32_t loff = uint32_t(lane >> 5) * uint32_t(a.logit_cap) + uint32_t(sl);
#pragma unroll 1
    for (int k = 0; k < 8; ++k) {   // heads 2k and 2k + 1 (not unrolled: fewer live registers)
      if (2 * k >= a.G) break;
      const int h = 2 * k + (lane >> 5);
      if (h < a.G && sok) lg_base[loff + uint32_t(2 * k) * uint32_t(a.logit_cap)] = lt[h * LP + (lane & 31)];
    }
  }
}

template <int D, bool VC, bool F8, bool APP>
__device__ __forceinline__ void mf_fetch(const MfCtx& x, int base, int lane, MfRaw<D, F8>& T) {
  if constexpr (F8) mf_load_f8<D, VC>(x, base, lane, T);
  else mf_load<D, VC, APP>(x, base, lane, T);
}

template <int D, bool F8>
__device__ __forceinline__ void mf_step(const AttnArgs& a, const MfCtx& x, int base, int lane, const u32x4* qv,
                                        float sc2, float* lg_base, float* lgs, uint16_t* vt, const MfRaw<D, F8>& T,
                                        MfState<D>& st) {
  mf_compute<D>(a, x, base, lane, qv, sc2, lg_base, lgs, vt, T, st);
}

// LG: logits requested.  Launches without them compile the logits path out, which
// keeps the register budget (a spill here costs far more than its few bytes).
// SEL > 0: the page view is selected in the launch (AttnArgs::sel), SEL keys per
// thread (up to 256 SEL pages).  H2O: the H2O decode step (AttnArgs::h2o): the
// logits go to LDS, then the unit's accumulate-then-evict runs in the block.
template <int D, bool VC, int OCC, bool F8, bool APP, bool LG, int SEL = 0, bool H2O = false>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(OCC, OCC)))
void attn_mfma_kernel(AttnArgs a) {
  static_assert(!(APP && F8), "the fused append writes bf16 rows");
  static_assert(SEL == 0 || (VC && !APP && !LG), "in-launch selection: page views, no fused append, no logits");
  static_assert(!H2O || (APP && LG && !VC && SEL == 0), "the H2O step: fused append, identity view, logits");
  __shared__ float lg_unit[H2O ? ATTN_H2O_LDS_LOGITS : 1];   // [head][slot], row pitch logit_cap
  __shared__ float h2o_lse[H2O ? 16 : 1];
  constexpr int PITCH = MF_TS + 4;          // u16 per transposed V row (72 bytes)
  constexpr int NDB = D / 16;
  constexpr int NKS = D / 32;
  static_assert(D == 64 || D == 128, "head width");
  __shared__ __align__(16) uint16_t vt_lds[MF_WAVES][D * PITCH];   // V tiles, then the wave merge
  __shared__ __align__(16) float lg_lds[LG ? MF_WAVES : 1][16 * (MF_TS + 4)];   // logits staging
  __shared__ u32x4 app_lds[APP ? 2 * (D / 8) : 1];   // the new row, parked during the tiles
  __shared__ float red_m[MF_WAVES][16], red_l[MF_WAVES][16];

  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int g = lane >> 4, c16 = lane & 15;
  const int unit = blockIdx.y, split = blockIdx.x;
  const int b = unit / a.Hkv, kvh = unit % a.Hkv;
  const int G = a.G;
  // A page / token view is chunked by its capacity, so the block can fetch its view
  // entries right away; slots past the view's length are masked.  The identity view
  // is chunked by seq_len.  With the LDS view cache (VC, page / token views only)
  // the entry loads depend on kernel arguments alone and are issued before the
  // lengths are read, so the two fetches overlap.
  const bool identity = !VC && a.view_idx == nullptr;
  constexpr int VPT = MF_VCACHE / 256;   // cached view entries per thread
  int ventry[VPT];
  int e0 = 0, s0, s1;
  // in-launch selection: the unit's page scores, loaded first (their addresses depend
  // on kernel arguments alone, so they overlap the length load), masked by the page
  // count once it is known
  float sraw[SEL > 0 ? SEL : 1];
  if constexpr (SEL > 0) {
    const float* srow = a.sel_score + size_t(unit) * a.sel_ncp;
#pragma unroll
    for (int j = 0; j < SEL; ++j) sraw[j] = srow[min(topk_reg_index<256, SEL>(j), a.sel_ncp - 1)];
  }
  if (VC) {
    const int n_slots = a.view_cap * a.gran;
    int chunk = (n_slots + a.splits - 1) / a.splits;
    chunk = (chunk + MF_TS - 1) / MF_TS * MF_TS;
    s0 = min(n_slots, split * chunk);
    s1 = min(n_slots, s0 + chunk);
    if constexpr (SEL == 0) {
      e0 = s0 >> a.gshift;
      const int e1 = s1 > s0 ? ((s1 - 1) >> a.gshift) + 1 : e0;
      const int32_t* vrow = a.view_idx + size_t(unit) * a.view_cap;
#pragma unroll
      for (int j = 0; j < VPT; ++j) {
        const int e = e0 + threadIdx.x + 256 * j;
        ventry[j] = e < e1 ? vrow[e] : -1;
      }
    }
  }
  const int len0 = min(a.seq_len[b], a.cap);
  int len = len0, tgt = -2, row_ticket = 0;
  if constexpr (SEL > 0) {   // the row the scoring launch appended
    if (len0 < a.cap) len = len0 + 1;
  }
  u32x4 app_row = {0, 0, 0, 0};   // this thread's 16 bytes of the new row, stored after the tiles
  if constexpr (APP) {
    // se_kv_append's rule, per unit
    const bool bump = a.slot == nullptr || a.slot[size_t(b) * a.Hkv] < 0;
    const int sl = a.slot != nullptr ? a.slot[unit] : -1;
    const int pos = sl >= 0 ? sl : len0;
    tgt = (pos >= 0 && pos < a.cap) ? pos : -2;
    if (bump && len0 < a.cap) len = len0 + 1;
    if (split == 0 && tgt >= 0 && threadIdx.x < 2 * (D / 8)) {   // the cache row, for later steps
      const bool isv = threadIdx.x >= D / 8;
      const int o = 8 * (isv ? threadIdx.x - D / 8 : threadIdx.x);
      app_row = ld16(static_cast<const uint16_t*>(isv ? a.v_new : a.k_new) + size_t(unit) * D + o);
    }
  }
  if (!VC) {
    const int n_slots = identity ? len : a.view_cap * a.gran;
    int chunk = (n_slots + a.splits - 1) / a.splits;
    chunk = (chunk + MF_TS - 1) / MF_TS * MF_TS;
    s0 = min(n_slots, split * chunk);
    s1 = min(n_slots, s0 + chunk);
  }

  // the view's slot count (selected in the launch: known after the selection)
  int s_valid = identity ? len : (SEL > 0 ? 0 : min(a.view_len[unit], a.view_cap) * a.gran);

  MfCtx x;
  const size_t ebytes = F8 ? 1 : 2;   // bytes per stored element
  x.ku = reinterpret_cast<const uint16_t*>(static_cast<const char*>(a.k) + size_t(unit) * a.cap * D * ebytes);
  x.vu = reinterpret_cast<const uint16_t*>(static_cast<const char*>(a.v) + size_t(unit) * a.cap * D * ebytes);
  x.ksc = F8 ? a.k_scale + size_t(unit) * a.cap : nullptr;
  x.vsc = F8 ? a.v_scale + size_t(unit) * a.cap : nullptr;
  x.len = len;
  x.s1 = min(s1, s_valid);
  x.gshift = a.gshift;
  x.identity = identity;
  x.e0 = e0;
  x.tgt = tgt;
  x.knew = APP ? static_cast<const uint16_t*>(a.k_new) + size_t(unit) * D : nullptr;
  x.vnew = APP ? static_cast<const uint16_t*>(a.v_new) + size_t(unit) * D : nullptr;
  x.vglob = (identity || SEL > 0) ? nullptr : a.view_idx + size_t(unit) * a.view_cap;

  // Q as the B operand: lane holds head c16, dims 32c + 8g .. 32c + 8g + 7 of k-step c
  // (FP8 tiles: dims 64 (c / 2) + 16 g + 8 (c % 2) on, the order of their K bytes)
  u32x4 qv[NKS];
  if (c16 < G) {
    const uint16_t* qh = (const uint16_t*)a.q + (size_t(b) * a.Hq + size_t(kvh) * G + c16) * D;
#pragma unroll
    for (int c = 0; c < NKS; ++c) qv[c] = ld16(qh + (F8 ? 64 * (c >> 1) + 16 * g + 8 * (c & 1) : 8 * g + 32 * c));
  } else {
#pragma unroll
    for (int c = 0; c < NKS; ++c) qv[c] = u32x4{0, 0, 0, 0};
  }
  int sel_len = 0;
  if constexpr (SEL > 0) {
    // the unit's top pages by score, ascending, straight into the view cache (the
    // V staging tiles are not in use yet and hold the selection's histograms)
    using SelShared = TopkRegSharedN<MF_WAVES, 2>;
    SelShared& tsh = *reinterpret_cast<SelShared*>(&vt_lds[0][0]);
    static_assert(sizeof(SelShared) <= sizeof(vt_lds), "selection scratch");
    const int npages = min((len + a.gran - 1) >> a.gshift, a.sel_ncp);
    uint32_t key[SEL > 0 ? SEL : 1];
#pragma unroll
    for (int j = 0; j < SEL; ++j) key[j] = topk_reg_index<256, SEL>(j) < npages ? ordered_bits(sraw[j]) : 0u;
    sel_len = block_topk_keys<256, SEL, SelShared>(key, npages, a.view_cap, mf_vcache, tsh);
  } else if (VC) {
#pragma unroll
    for (int j = 0; j < VPT; ++j)
      if (threadIdx.x + 256 * j < MF_VCACHE) mf_vcache[threadIdx.x + 256 * j] = ventry[j];
  }
  __syncthreads();   // view cache ready
  if constexpr (SEL > 0) {
    s_valid = min(sel_len, a.view_cap) * a.gran;
    x.s1 = min(s1, s_valid);
  }
  if (SEL > 0 && split == 0 && a.sel_view != nullptr) {
    for (int i = threadIdx.x; i < a.view_cap; i += 256) a.sel_view[size_t(unit) * a.view_cap + i] = mf_vcache[i];
    if (threadIdx.x == 0) a.sel_vlen[unit] = sel_len;
  }

  const float sc2 = a.scale * LOG2E;
  MfState<D> st;
  st.m2 = -INFINITY;
  st.lsum = 0.f;
#pragma unroll
  for (int i = 0; i < NDB; ++i) st.o[i] = f32x4{0.f, 0.f, 0.f, 0.f};
  uint16_t* vt = vt_lds[w];   // row pitch PITCH, D rows
  float* lgs = LG ? lg_lds[w] : nullptr;
  // the group's first logits row (head h at + h * logit_cap), or null: wave-uniform
  float* lg_base = H2O ? lg_unit : LG ? a.logits + (size_t(b) * a.Hq + size_t(kvh) * G) * a.logit_cap : nullptr;

  // This wave's tiles are w, w + 4, ...  The steady-state loop runs only while
  // every tile it prefetches exists: its loads are unconditional and an
  // iteration ends with the same tiles in flight as it began, so the compiler's
  // wait counts stay exact (computing a tile waits only for that tile's loads).
  // The last two to four tiles are drained without further prefetch, so no wave
  // ends waiting on a load it will not use.
  const int ntiles = (s1 - s0 + MF_TS - 1) / MF_TS;
  const int nmine = w < ntiles ? (ntiles - w + MF_WAVES - 1) / MF_WAVES : 0;
  constexpr int STEP = MF_WAVES * MF_TS;   // slots between this wave's consecutive tiles
  const int first = s0 + w * MF_TS;
  // the new row's 16 bytes per thread wait in LDS while the tiles run (written once
  // the first tile's loads are out, so that its wait delays none of them): four
  // fewer registers held across the loop
  const bool app_mine = APP && split == 0 && tgt >= 0 && threadIdx.x < 2 * (D / 8);
  auto park_app_row = [&]() {
    if (app_mine) app_lds[threadIdx.x] = app_row;
  };
  if (OCC == 1) {
    MfRaw<D, F8> T0, T1, T2;               // two tiles in flight while a third is computed
    if (nmine == 0) {
      park_app_row();
    } else if (nmine == 1) {
      mf_fetch<D, VC, F8, APP>(x, first, lane, T0);
      park_app_row();
      mf_step<D, F8>(a, x, first, lane, qv, sc2, lg_base, lgs, vt, T0, st);
    } else {
      mf_fetch<D, VC, F8, APP>(x, first, lane, T0);
      mf_fetch<D, VC, F8, APP>(x, first + STEP, lane, T1);
      park_app_row();
      int i = 0;
      for (; i + 4 < nmine; i += 3) {      // T0 = tile i, T1 = tile i + 1 in flight
        const int b0 = first + i * STEP;
        mf_fetch<D, VC, F8, APP>(x, b0 + 2 * STEP, lane, T2);
        mf_step<D, F8>(a, x, b0, lane, qv, sc2, lg_base, lgs, vt, T0, st);
        mf_fetch<D, VC, F8, APP>(x, b0 + 3 * STEP, lane, T0);
        mf_step<D, F8>(a, x, b0 + STEP, lane, qv, sc2, lg_base, lgs, vt, T1, st);
        mf_fetch<D, VC, F8, APP>(x, b0 + 4 * STEP, lane, T1);
        mf_step<D, F8>(a, x, b0 + 2 * STEP, lane, qv, sc2, lg_base, lgs, vt, T2, st);
      }
      const int r = nmine - i;             // 2, 3 or 4 tiles left
      const int b0 = first + i * STEP;
      if (r >= 3) mf_fetch<D, VC, F8, APP>(x, b0 + 2 * STEP, lane, T2);
      mf_step<D, F8>(a, x, b0, lane, qv, sc2, lg_base, lgs, vt, T0, st);
      if (r == 4) mf_fetch<D, VC, F8, APP>(x, b0 + 3 * STEP, lane, T0);
      mf_step<D, F8>(a, x, b0 + STEP, lane, qv, sc2, lg_base, lgs, vt, T1, st);
      if (r >= 3) mf_step<D, F8>(a, x, b0 + 2 * STEP, lane, qv, sc2, lg_base, lgs, vt, T2, st);
      if (r == 4) mf_step<D, F8>(a, x, b0 + 3 * STEP, lane, qv, sc2, lg_base, lgs, vt, T0, st);
    }
  } else {
    MfRaw<D, F8> T0, T1;                   // one tile in flight while the other is computed
    if (nmine == 0) park_app_row();
    if (nmine > 0) {
      mf_fetch<D, VC, F8, APP>(x, first, lane, T0);
      park_app_row();
      int i = 0;
      for (; i + 2 < nmine; i += 2) {      // T0 = tile i in flight
        const int b0 = first + i * STEP;
        mf_fetch<D, VC, F8, APP>(x, b0 + STEP, lane, T1);
        mf_step<D, F8>(a, x, b0, lane, qv, sc2, lg_base, lgs, vt, T0, st);
        mf_fetch<D, VC, F8, APP>(x, b0 + 2 * STEP, lane, T0);
        mf_step<D, F8>(a, x, b0 + STEP, lane, qv, sc2, lg_base, lgs, vt, T1, st);
      }
      const int b0 = first + i * STEP;     // one or two tiles left
      if (i + 1 < nmine) {
        mf_fetch<D, VC, F8, APP>(x, b0 + STEP, lane, T1);
        mf_step<D, F8>(a, x, b0, lane, qv, sc2, lg_base, lgs, vt, T0, st);
        mf_step<D, F8>(a, x, b0 + STEP, lane, qv, sc2, lg_base, lgs, vt, T1, st);
      } else {
        mf_step<D, F8>(a, x, b0, lane, qv, sc2, lg_base, lgs, vt, T0, st);
      }
    }
  }

  if ((APP || SEL > 0) && threadIdx.x == 0) {
    // every block of the batch row takes a ticket, long after it read the old length
    // (issued here, not up front, so that no tile's loads wait for its return); the
    // last one stores the new length at the end
    row_ticket = __hip_atomic_fetch_add(a.row_ctr + b, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  if (app_mine) {   // its load went out before the tiles
    const bool isv = threadIdx.x >= D / 8;
    const int o = 8 * (isv ? threadIdx.x - D / 8 : threadIdx.x);
    *reinterpret_cast<u32x4*>(static_cast<uint16_t*>(isv ? a.v_w : a.k_w) + (size_t(unit) * a.cap + tgt) * D + o) =
        app_lds[threadIdx.x];
  }
  // H2O: the slots' positions and scores, loaded now so that their round trip overlaps
  // the wave and head merges below (nothing in this launch writes them before they are
  // used, but for the slot past the occupied ones, which no thread loads)
  constexpr int HE = ATTN_H2O_SLOTS_PER_THREAD;
  int h2o_p[H2O ? HE : 1];
  float h2o_sc[H2O ? HE : 1];
  if constexpr (H2O) {
    const int32_t* pos = a.h2o_pos + size_t(unit) * a.cap;
    const float* acc = a.h2o_acc + size_t(unit) * a.cap;
#pragma unroll
    for (int j = 0; j < HE; ++j) {
      const int sl = max(min(j * 256 + int(threadIdx.x), len - 1), 0);
      h2o_p[j] = pos[sl];
      h2o_sc[j] = acc[sl];
    }
  }
  // ---- merge the waves of the block: per head, the waves' (max, sum) and
  // outputs [wave][head][dim] (row pitch D + 4) go through LDS; a thread then
  // owns four consecutive dims of one head.
  float lsum = st.lsum;
  lsum = rows4_sum(lsum);
  constexpr int OP = D + 4;
  __syncthreads();
  float* red_o = reinterpret_cast<float*>(&vt_lds[0][0]);
  static_assert(MF_WAVES * 16 * OP * sizeof(float) <= sizeof(vt_lds), "reduction buffer");
  if (g == 0) { red_m[w][c16] = st.m2; red_l[w][c16] = lsum; }
#pragma unroll
  for (int db = 0; db < NDB; ++db)
    *reinterpret_cast<f32x4*>(red_o + (w * 16 + c16) * OP + 16 * db + 4 * g) = st.o[db];
  __syncthreads();
  float* pml = a.part_ml + (size_t(unit) * a.splits + split) * G * 2;
  float* po = a.part_o + (size_t(unit) * a.splits + split) * G * D;
  const bool single = a.splits == 1;
  for (int idx = threadIdx.x * 4; idx < G * D; idx += 256 * 4) {
    const int h = idx / D, d0 = idx % D;
    float M = red_m[0][h];
#pragma unroll
    for (int ww = 1; ww < MF_WAVES; ++ww) M = fmaxf(M, red_m[ww][h]);
    float L = 0.f;
    f32x4 O = {0.f, 0.f, 0.f, 0.f};
    if (M != -INFINITY) {
#pragma unroll
      for (int ww = 0; ww < MF_WAVES; ++ww) {
        const float mw = red_m[ww][h];
        if (mw != -INFINITY) {
          const float f = ex2(mw - M);
          L += f * red_l[ww][h];
          O += f * *reinterpret_cast<const f32x4*>(red_o + (ww * 16 + h) * OP + d0);
        }
      }
    }
    const float Mn = M == -INFINITY ? -INFINITY : M * 0.6931471805599453f;   // log2 -> natural units
    if (single) {
      const size_t row = size_t(b) * a.Hq + size_t(kvh) * G + h;
      const float inv = L > 0.f ? 1.f / L : 0.f;
      *reinterpret_cast<f32x4*>(a.out + row * D + d0) = O * inv;
      if (d0 == 0 && a.lse != nullptr) a.lse[row] = L > 0.f ? Mn + logf(L) : -INFINITY;
      if (H2O && d0 == 0) h2o_lse[h] = L > 0.f ? Mn + logf(L) : -INFINITY;
    } else if (a.fused) {
      st_dev2(po + h * D + d0, O[0], O[1]);
      st_dev2(po + h * D + d0 + 2, O[2], O[3]);
      if (d0 == 0) st_dev2(pml + 2 * h, Mn, L);
    } else {
      *reinterpret_cast<float2*>(po + h * D + d0) = make_float2(O[0], O[1]);
      *reinterpret_cast<float2*>(po + h * D + d0 + 2) = make_float2(O[2], O[3]);
      if (d0 == 0) *reinterpret_cast<float2*>(pml + 2 * h) = make_float2(Mn, L);
    }
  }
  if (a.fused) {
    int* ctr = a.counters + unit * ATTN_MAX_HG;
    if (attn_split_done(ctr, a.splits)) attn_merge_splits<256>(a, unit, 0, G, ctr);
  }
  if constexpr (H2O) {
    // the H2O accumulate-then-evict of this unit, as se_h2o_accumulate_evict (h2o_reg_kernel)
    // computes it from the logits and lse of the attention: the same operations in the same
    // order, with the logits read from LDS instead of memory
    __syncthreads();   // every tile's logits and the heads' lse are in LDS
    __shared__ int h2o_cnt[MF_WAVES], h2o_slot[MF_WAVES];
    __shared__ uint32_t h2o_hi[MF_WAVES], h2o_lo[MF_WAVES];
    const int n = len;
    int32_t* pos = a.h2o_pos + size_t(unit) * a.cap;
    float* acc = a.h2o_acc + size_t(unit) * a.cap;
    const int in = a.slot != nullptr ? a.slot[unit] : -1;
    const int ns = in >= 0 ? in : n - 1;   // the slot that received the token at cur_pos
    if (threadIdx.x == 0 && ns >= n && ns < a.cap) { pos[ns] = a.h2o_cur; acc[ns] = 0.f; }
    int (&p)[HE] = h2o_p;
    float (&sc)[HE] = h2o_sc;
#pragma unroll
    for (int j = 0; j < HE; ++j) {
      const int sl = j * 256 + threadIdx.x;
      if (sl >= n) { p[j] = -1; sc[j] = 0.f; }
      if (sl == ns) { p[j] = a.h2o_cur; sc[j] = 0.f; }
    }
    // heads in ascending order.  A head's logits are read unconditionally (clamped
    // slot) and together, so one LDS wait covers them, and each sum takes its term only
    // for an occupied slot (a per-lane branch around each read had made every read a
    // waited LDS round trip of its own)
    static_assert(sizeof(h2o_lse) / sizeof(h2o_lse[0]) == 16, "at most 16 heads per KV head");
#pragma unroll
    for (int hh = 0; hh < 16; ++hh) {
      if (hh >= G) break;
      const float l = h2o_lse[hh];
      if (l == -INFINITY) continue;
      float lv[HE];
#pragma unroll
      for (int j = 0; j < HE; ++j) lv[j] = lg_unit[hh * a.logit_cap + min(j * 256 + int(threadIdx.x), a.logit_cap - 1)];
#pragma unroll
      for (int j = 0; j < HE; ++j) {
        const float e = h2o_exp(lv[j] - l);
        sc[j] = p[j] >= 0 ? sc[j] + e : sc[j];
      }
    }
    int cnt = 0;
#pragma unroll
    for (int j = 0; j < HE; ++j) {
      const int sl = j * 256 + threadIdx.x;
      if (sl < n) {
        if (sl == ns) pos[sl] = a.h2o_cur;
        if (p[j] >= 0) acc[sl] = sc[j];
        else if (sl == ns) acc[sl] = 0.f;
        cnt += p[j] >= 0;
      }
    }
    cnt = wave_sum_i(cnt);
    if (lane == 0) h2o_cnt[w] = cnt;
    __syncthreads();
    const int occupied = h2o_cnt[0] + h2o_cnt[1] + h2o_cnt[2] + h2o_cnt[3];
    if (occupied <= a.h2o_heavy + a.h2o_recent) {
      if (threadIdx.x == 0) a.h2o_evict[unit] = -1;
    } else {
      // argmin of (score, position) over the slots outside the recent window
      uint32_t bh = ~0u, bl = ~0u;
      int bs = -1;
#pragma unroll
      for (int j = 0; j < HE; ++j) {
        const int sl = j * 256 + threadIdx.x;
        if (sl < n && p[j] >= 0 && p[j] <= a.h2o_cur - a.h2o_recent) {
          const uint32_t hkey = ordered_bits(sc[j]), lkey = uint32_t(p[j]);
          if (hkey < bh || (hkey == bh && lkey < bl)) { bh = hkey; bl = lkey; bs = sl; }
        }
      }
      const uint32_t wh = wave_last(wave_incl_scan_dpp(bh, ~0u, [](uint32_t x, uint32_t y) { return x < y ? x : y; }));
      const uint32_t wl = wave_last(wave_incl_scan_dpp(bh == wh ? bl : ~0u, ~0u,
                                                       [](uint32_t x, uint32_t y) { return x < y ? x : y; }));
      const uint64_t hit = __ballot(bh == wh && bl == wl && bs >= 0);
      const int wsl = hit ? __builtin_amdgcn_readlane(bs, __ffsll((unsigned long long)hit) - 1) : -1;
      if (lane == 0) { h2o_hi[w] = wh; h2o_lo[w] = wl; h2o_slot[w] = wsl; }
      __syncthreads();
      if (threadIdx.x == 0) {
        uint32_t kh = h2o_hi[0], kl = h2o_lo[0];
        int ev = h2o_slot[0];
        for (int i = 1; i < MF_WAVES; ++i)
          if (h2o_slot[i] >= 0 && (ev < 0 || h2o_hi[i] < kh || (h2o_hi[i] == kh && h2o_lo[i] < kl))) {
            kh = h2o_hi[i]; kl = h2o_lo[i]; ev = h2o_slot[i];
          }
        if (ev >= 0) { pos[ev] = -1; acc[ev] = 0.f; }
        a.h2o_evict[unit] = ev;
      }
    }
  }
  if ((APP || SEL > 0) && threadIdx.x == 0 && row_ticket == a.Hkv * a.splits - 1) {   // every block of the row has read it
    if (len != len0) a.seq_len_w[b] = len;
    ticket_reset(a.row_ctr + b);
  }
}

bool attn_mfma_supported(const AttnArgs& a) {
  return a.dtype == SE_BF16 && !a.latent && (a.Dk == 128 || a.Dk == 64) && a.Dv == a.Dk && a.G <= 16 &&
         (a.view_idx == nullptr || a.gshift >= 0) && a.cap <= (1 << 30) / a.Dk;
}

// Long views: two blocks per CU (512 blocks) as long as every split keeps at
// least 1024 slots; otherwise one block per CU (256 blocks) with at least four
// tiles per block.
int attn_mfma_auto_splits(int units, int slots) {
  int s = (512 + units - 1) / units;
  s = std::max(1, std::min(s, slots / 1024));
  if (units * s < 256) s = std::max(1, std::min((256 + units - 1) / units, (slots + 4 * MF_TS - 1) / (4 * MF_TS)));
  return std::min(s, 256);
}

template <int D, bool VC, int OCC, bool F8, bool APP>
static void mf_launch(const AttnArgs& a, dim3 grid, hipStream_t s) {
  if (a.logits != nullptr)
    hipLaunchKernelGGL((attn_mfma_kernel<D, VC, OCC, F8, APP, true>), grid, dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL((attn_mfma_kernel<D, VC, OCC, F8, APP, false>), grid, dim3(256), 0, s, a);
}

// Keys per thread of the in-launch page selection for sel_ncp pages (0: too many).
int attn_mfma_sel_keys(int ncp) { return ncp <= 256 * 4 ? 4 : ncp <= 256 * 9 ? 9 : ncp <= 256 * 16 ? 16 : 0; }

se_status launch_attn_mfma(const AttnArgs& a, hipStream_t s) {
  dim3 grid(a.splits, a.B * a.Hkv);
  if (a.h2o) {   // the H2O decode step: fused append, identity view, logits in LDS, one split
    if (a.splits != 1 || !a.app || a.view_idx != nullptr) return SE_ERR_UNSUPPORTED;
    if (a.Dk == 128)
      hipLaunchKernelGGL((attn_mfma_kernel<128, false, 2, false, true, true, 0, true>), grid, dim3(256), 0, s, a);
    else
      hipLaunchKernelGGL((attn_mfma_kernel<64, false, 1, false, true, true, 0, true>), grid, dim3(256), 0, s, a);
    return launch_status();
  }
  if (a.sel) {   // page views selected in the launch (the Quest decode step, bf16 or FP8 rows)
#define SE_SEL(DD, OO, FF, EE) hipLaunchKernelGGL((attn_mfma_kernel<DD, true, OO, FF, false, false, EE>), grid, \
                                                  dim3(256), 0, s, a)
#define SE_SEL_E(DD, OO, FF)                                                                                   \
  if (e == 4) SE_SEL(DD, OO, FF, 4); else if (e == 9) SE_SEL(DD, OO, FF, 9); else if (e == 16) SE_SEL(DD, OO, FF, 16); \
  else return SE_ERR_UNSUPPORTED;
    const int e = attn_mfma_sel_keys(a.sel_ncp);
    if (a.Dk == 128) {
      if (a.fp8) { SE_SEL_E(128, 2, true) } else { SE_SEL_E(128, 2, false) }
    } else {
      if (a.fp8) { SE_SEL_E(64, 1, true) } else { SE_SEL_E(64, 1, false) }
    }
#undef SE_SEL_E
#undef SE_SEL
    return launch_status();
  }
  // entries one block reads: its chunk of slots divided by the granularity (+2 for straddled entries)
  const int slots = a.view_idx ? a.view_cap * a.gran : 0;
  int chunk = (slots + a.splits - 1) / a.splits;
  chunk = (chunk + MF_TS - 1) / MF_TS * MF_TS;
  const bool vc = a.view_idx != nullptr && chunk / a.gran + 2 <= MF_VCACHE;
#define SE_MF_LAUNCH(DD, VV, OO, FF, AA) mf_launch<DD, VV, OO, FF, AA>(a, grid, s)
#define SE_MF_D(FF, AA)                                                                              \
  if (a.Dk == 128) {                                                                                 \
    if (vc) SE_MF_LAUNCH(128, true, 2, FF, AA); else SE_MF_LAUNCH(128, false, 2, FF, AA);            \
  } else {                                                                                           \
    if (vc) SE_MF_LAUNCH(64, true, 1, FF, AA); else SE_MF_LAUNCH(64, false, 1, FF, AA);              \
  }
  if (a.app) {   // the fused append writes bf16 rows
    SE_MF_D(false, true)
  } else if (a.fp8) {
    SE_MF_D(true, false)
  } else {
    SE_MF_D(false, false)
  }
#undef SE_MF_D
#undef SE_MF_LAUNCH
  return launch_status();
}

}  // namespace se
