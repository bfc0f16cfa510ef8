// MLA latent decode attention on MFMA (gfx950, v_mfma_f32_16x16x32_bf16).
//
// Every head of a batch row reads the same 576-wide latent row per token: the
// key is the whole row (512 latent + 64 rope columns) and the value is its
// first 512 columns (SparseEngine pages: GLM-4.7-Flash is an MLA model and
// the engine supports MLA beside GQA).  Each row is read from HBM once and
// feeds both products:
//   S^T[token][head] = C[token][:] . Q[head][:]          (576-deep)
//   O^T[dim][head]  += C[token][dim]^T . P^T[token][head] (dims 0..511)
//
// Groups of up to 16 heads (attn_mla_kernel): 8 waves per (unit, split, head
// group), tiles of 128 view slots.  Wave w scores slots 16w..16w+15 of a tile
// over all 576 columns (K rows go from HBM straight into A-operand registers;
// Q is staged once in LDS in B-operand order), and owns output dims
// 64w..64w+63 for all heads: it loads those 64 columns of all 128 rows a second
// time in a four-token-per-lane order (an L2 hit), which a v_perm transpose
// turns into V^T in a wave-private LDS tile.  Softmax state is shared through
// LDS: the waves post their per-head maxima, all of them take the same tile
// maximum and make the same (lazy, 2^8-margin) rescaling decision, and each
// wave posts P of its own slots as bf16 hi + lo pairs that every wave then reads
// as the B operand.  The next tile's rows and value columns are issued together
// at the end of a tile.
//
// Groups of 17..32 heads take attn_mla_pf_kernel below: 64-slot tiles, the next
// tile's rows in flight in registers while the current one is used, and the
// values read from LDS copies of the rows already loaded.
//
// Each split stores a partial (max, sum, output), which the combine kernel
// merges (or, for small partials, the block finishing the last split).
//
// SEL > 0 (attn_mla_pf_kernel, the fused Quest decode step over latent rows):
// the page view is selected inside the launch from the page scores the scoring
// launch wrote (every block of a unit selects the same pages: the register
// top-k of block_topk_keys, SEL keys per thread), the scores' loads going out
// with q's; the row appended by the scoring launch is counted, and the last
// block of a batch row stores the new length.
#include "attn_common.hpp"
#include "mfma_util.hpp"

#include <type_traits>

namespace se {

constexpr int ML_DK = 576, ML_DV = 512;
constexpr int ML_WAVES = 8, ML_THREADS = ML_WAVES * 64;
constexpr int ML_TS = 128;                      // slots per tile (16 per wave)
constexpr int ML_NKS = ML_DK / 32;              // 18 k-steps of the score product
constexpr int ML_DW = ML_DV / ML_WAVES;         // 64 output dims per wave
constexpr int ML_PITCH = 32 + 4;                // u16 per transposed V row
constexpr int ML_VCACHE = 1024;                 // view entries cached per block
constexpr float ML_MARGIN = 8.f;                // log2 units

// LDS carve-up (bytes); the output transpose at the end reuses the whole area.
constexpr int ML_Q_BYTES = ML_NKS * 2 * 64 * 16;                 // 36864
constexpr int ML_P_BYTES = (ML_TS / 32) * 2 * 2 * 2 * 64 * 8;     // 16384: [kstep][half][hb][hi/lo][lane] uint2
constexpr int ML_VT_BYTES = ML_WAVES * ML_DW * ML_PITCH * 2;      // 36864
constexpr int ML_OB_PITCH = ML_DW + 4;                            // floats per head row of the output transpose
constexpr int ML_OB_BYTES = ML_WAVES * 32 * ML_OB_PITCH * 4;      // 69632
constexpr int ML_MAIN_BYTES = ML_Q_BYTES + ML_P_BYTES + ML_VT_BYTES;
constexpr int ML_LDS_BYTES = ML_MAIN_BYTES > ML_OB_BYTES ? ML_MAIN_BYTES : ML_OB_BYTES;

struct MlCtx {
  const uint16_t* cu;   // latent rows of the unit
  int len, s1, gshift, e0;
  bool identity;
};

__device__ __forceinline__ int ml_token(const MlCtx& x, const int32_t* vcache, int s) {
  int t;
  if (x.identity) {
    t = s;
  } else {
    // read unconditionally (clamped index): no branch, no wait per lookup
    const int pv = vcache[min(max((s >> x.gshift) - x.e0, 0), ML_VCACHE - 1)];
    const int page = s < x.s1 ? pv : -1;
    t = page < 0 ? -1 : (page << x.gshift) + (s & ((1 << x.gshift) - 1));
  }
  return (s < x.s1 && t >= 0 && t < x.len) ? t : -1;
}

// K rows of this wave's 16 slots (A operand: lane holds row c16, columns 32c + 8g .. + 7).
__device__ __forceinline__ int ml_load_k(const MlCtx& x, const int32_t* vcache, int tb, int w, int lane,
                                         u32x4 (&k)[ML_NKS]) {
  const int tk = ml_token(x, vcache, tb + 16 * w + (lane & 15));
  // unconditional loads keep the wait counts exact; a slot without a token reads row 0
  const uint32_t r = uint32_t(max(tk, 0)) * ML_DK + 8 * (lane >> 4);
#pragma unroll
  for (int c = 0; c < ML_NKS; ++c) k[c] = ld16(x.cu + r + 32 * c);
  return tk;
}

// This wave's 64 value columns of all 128 slots: lane holds slots 32p + 4(lane >> 3) + r,
// columns 64w + 8(lane & 7) .. + 7.
__device__ __forceinline__ void ml_load_v(const MlCtx& x, const int32_t* vcache, int tb, int w, int lane,
                                          u32x4 (&v)[4][4]) {
  const int qq = lane >> 3, col = ML_DW * w + 8 * (lane & 7);
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    const int sq = tb + 32 * p + 4 * qq;
    int vt[4];
    if (x.identity || x.gshift >= 2) {   // a 4-aligned slot quad stays inside one view entry
      const int t0 = ml_token(x, vcache, sq);
#pragma unroll
      for (int r = 0; r < 4; ++r) vt[r] = (t0 >= 0 && sq + r < x.s1 && t0 + r < x.len) ? t0 + r : -1;
    } else {
#pragma unroll
      for (int r = 0; r < 4; ++r) vt[r] = ml_token(x, vcache, sq + r);
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) v[p][r] = ld16(x.cu + uint32_t(max(vt[r], 0)) * ML_DK + col);
  }
}

template <int NHB>
__global__ __launch_bounds__(ML_THREADS) void attn_mla_kernel(AttnArgs a) {
  __shared__ __align__(16) unsigned char lds[ML_LDS_BYTES];
  __shared__ float wmax[ML_WAVES][32];
  __shared__ float wsum[ML_WAVES][32];
  __shared__ int32_t vcache[ML_VCACHE];
  u32x4* qs = reinterpret_cast<u32x4*>(lds);                                    // [NKS][hb][lane]
  uint2* ps = reinterpret_cast<uint2*>(lds + ML_Q_BYTES);                       // [kstep][half][hb][hl][lane]
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int g = lane >> 4, c16 = lane & 15;
  uint16_t* vt = reinterpret_cast<uint16_t*>(lds + ML_Q_BYTES + ML_P_BYTES) + w * ML_DW * ML_PITCH;

  const int unit = blockIdx.y, split = blockIdx.x, hg = blockIdx.z;
  const int b = unit / a.Hkv, kvh = unit % a.Hkv;
  const int G = a.G, h0 = 32 * hg;                 // heads h0 .. h0 + 31 of the group
  const bool identity = a.view_idx == nullptr;
  const int len = min(a.seq_len[b], a.cap);
  const int n_slots = identity ? len : a.view_cap * a.gran;
  const int s_valid = identity ? len : min(a.view_len[unit], a.view_cap) * a.gran;
  int chunk = (n_slots + a.splits - 1) / a.splits;
  chunk = (chunk + ML_TS - 1) / ML_TS * ML_TS;
  const int s0 = min(n_slots, split * chunk), s1 = min(n_slots, s0 + chunk);

  MlCtx x;
  x.cu = (const uint16_t*)a.k + size_t(unit) * a.cap * ML_DK;
  x.len = len;
  x.s1 = min(s1, s_valid);
  x.gshift = a.gshift;
  x.identity = identity;
  x.e0 = 0;
  if (!identity) {
    const int32_t* vrow = a.view_idx + size_t(unit) * a.view_cap;
    const int e0 = s0 >> a.gshift, e1 = s1 > s0 ? ((s1 - 1) >> a.gshift) + 1 : e0;
    for (int e = e0 + threadIdx.x; e < e1; e += ML_THREADS) vcache[e - e0] = vrow[e];
    x.e0 = e0;
  }
  // Q in B-operand order: entry (c, hb, lane) = head h0 + 16 hb + (lane & 15), columns 32c + 8(lane >> 4) .. + 7
  for (int i = threadIdx.x; i < ML_NKS * NHB * 64; i += ML_THREADS) {
    const int l = i & 63, hb = (i >> 6) % NHB, c = i / (64 * NHB);
    const int h = h0 + 16 * hb + (l & 15);
    u32x4 val = {0u, 0u, 0u, 0u};
    if (h < G) val = ld16((const uint16_t*)a.q + (size_t(b) * a.Hq + size_t(kvh) * G + h) * ML_DK + 32 * c + 8 * (l >> 4));
    qs[(c * 2 + hb) * 64 + l] = val;
  }
  __syncthreads();

  const float sc2 = a.scale * LOG2E;
  f32x4 o[ML_DW / 16][NHB];
#pragma unroll
  for (int db = 0; db < ML_DW / 16; ++db)
#pragma unroll
    for (int hb = 0; hb < NHB; ++hb) o[db][hb] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m2[NHB], lsum[NHB];
#pragma unroll
  for (int hb = 0; hb < NHB; ++hb) { m2[hb] = -INFINITY; lsum[hb] = 0.f; }

  const int ntiles = (s1 - s0 + ML_TS - 1) / ML_TS;
  u32x4 kr[ML_NKS];
  u32x4 vr[4][4];
  int tk = ml_load_k(x, vcache, s0, w, lane, kr);
  ml_load_v(x, vcache, s0, w, lane, vr);

  for (int it = 0; it < ntiles; ++it) {
    const int tb = s0 + it * ML_TS;
    // ---- scores of this wave's 16 slots for the group's heads
    f32x4 sa[NHB];
#pragma unroll
    for (int hb = 0; hb < NHB; ++hb) sa[hb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int c = 0; c < ML_NKS; ++c)
#pragma unroll
      for (int hb = 0; hb < NHB; ++hb) sa[hb] = mfma_bf16_16x16x32(kr[c], qs[(c * 2 + hb) * 64 + lane], sa[hb]);
    const uint64_t valid = __ballot(tk >= 0);

    float sv[NHB][4];
#pragma unroll
    for (int hb = 0; hb < NHB; ++hb)
#pragma unroll
      for (int i = 0; i < 4; ++i) sv[hb][i] = ((valid >> (4 * g + i)) & 1) ? sa[hb][i] * sc2 : -INFINITY;
    if (a.logits != nullptr) {
#pragma unroll
      for (int hb = 0; hb < NHB; ++hb) {
        const int h = h0 + 16 * hb + c16;
        if (h < G) {
          float* row = a.logits + (size_t(b) * a.Hq + size_t(kvh) * G + h) * a.logit_cap;
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int s = tb + 16 * w + 4 * g + i;
            if (s < x.s1 && s < a.logit_cap) row[s] = ((valid >> (4 * g + i)) & 1) ? sa[hb][i] * a.scale : -INFINITY;
          }
        }
      }
    }
    // ---- tile maximum per head, shared by all waves
#pragma unroll
    for (int hb = 0; hb < NHB; ++hb) {
      float m = fmaxf(fmaxf(sv[hb][0], sv[hb][1]), fmaxf(sv[hb][2], sv[hb][3]));
      m = rows4_max(m);
      if (g == 0) wmax[w][16 * hb + c16] = m;
    }
    __syncthreads();
#pragma unroll
    for (int hb = 0; hb < NHB; ++hb) {
      float tmax = wmax[0][16 * hb + c16];
#pragma unroll
      for (int ww = 1; ww < ML_WAVES; ++ww) tmax = fmaxf(tmax, wmax[ww][16 * hb + c16]);
      // every wave sees the same maxima and takes the same decision
      const bool grow = tmax > m2[hb] + ML_MARGIN;
      if (__ballot(grow) != 0) {
        const float mnew = grow ? tmax : m2[hb];
        const float alpha = (grow && m2[hb] != -INFINITY) ? ex2(m2[hb] - mnew) : 1.f;
        lsum[hb] *= alpha;
#pragma unroll
        for (int db = 0; db < ML_DW / 16; ++db) o[db][hb] *= alpha;
        m2[hb] = mnew;
      }
      const float mref = m2[hb] == -INFINITY ? 0.f : m2[hb];
      float p[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        p[i] = ex2(sv[hb][i] - mref);   // 0 for masked slots, at most 2^8 otherwise
        lsum[hb] += p[i];
      }
      uint2 hi, lo;
      hi.x = pack_bf16(p[0], p[1]);
      hi.y = pack_bf16(p[2], p[3]);
      lo.x = pack_bf16(p[0] - bf16x2_lo_f32(hi.x), p[1] - bf16x2_hi_f32(hi.x));
      lo.y = pack_bf16(p[2] - bf16x2_lo_f32(hi.y), p[3] - bf16x2_hi_f32(hi.y));
      // slots 16w + 4g + i = k-step w / 2, half w % 2
      ps[((((w >> 1) * 2 + (w & 1)) * 2 + hb) * 2 + 0) * 64 + lane] = hi;
      ps[((((w >> 1) * 2 + (w & 1)) * 2 + hb) * 2 + 1) * 64 + lane] = lo;
    }
    __syncthreads();

    // ---- O^T += V^T P^T over the tile's four 32-slot k-steps
    const int qq = lane >> 3, ch = lane & 7;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        const uint32_t w0 = vr[j][0][m], w1 = vr[j][1][m], w2 = vr[j][2][m], w3 = vr[j][3][m];
        uint2 lo2, hi2;
        lo2.x = lo16_pair(w0, w1);
        lo2.y = lo16_pair(w2, w3);
        hi2.x = hi16_pair(w0, w1);
        hi2.y = hi16_pair(w2, w3);
        *reinterpret_cast<uint2*>(vt + (8 * ch + 2 * m) * ML_PITCH + 4 * qq) = lo2;
        *reinterpret_cast<uint2*>(vt + (8 * ch + 2 * m + 1) * ML_PITCH + 4 * qq) = hi2;
      }
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
      u32x4 ph[NHB], pl[NHB];
#pragma unroll
      for (int hb = 0; hb < NHB; ++hb) {
        const uint2 h0v = ps[((((j * 2 + 0) * 2 + hb) * 2) + 0) * 64 + lane];
        const uint2 h1v = ps[((((j * 2 + 1) * 2 + hb) * 2) + 0) * 64 + lane];
        const uint2 l0v = ps[((((j * 2 + 0) * 2 + hb) * 2) + 1) * 64 + lane];
        const uint2 l1v = ps[((((j * 2 + 1) * 2 + hb) * 2) + 1) * 64 + lane];
        ph[hb] = u32x4{h0v.x, h0v.y, h1v.x, h1v.y};
        pl[hb] = u32x4{l0v.x, l0v.y, l1v.x, l1v.y};
      }
#pragma unroll
      for (int db = 0; db < ML_DW / 16; ++db) {
        const uint16_t* row = vt + (16 * db + c16) * ML_PITCH;
        const uint2 x0 = *reinterpret_cast<const uint2*>(row + 4 * g);
        const uint2 x1 = *reinterpret_cast<const uint2*>(row + 16 + 4 * g);
        const u32x4 av = {x0.x, x0.y, x1.x, x1.y};
#pragma unroll
        for (int hb = 0; hb < NHB; ++hb) {
          o[db][hb] = mfma_bf16_16x16x32(av, ph[hb], o[db][hb]);
          o[db][hb] = mfma_bf16_16x16x32(av, pl[hb], o[db][hb]);
        }
      }
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    }
    // next tile: its rows and this wave's value columns of them go out together, so
    // the column reads (rows other waves fetch) meet those rows in flight or fresh in
    // L2; fetched half a tile apart, a tile step's rows (~4.7 MB per XCD) evicted them
    tk = ml_load_k(x, vcache, tb + ML_TS, w, lane, kr);
    ml_load_v(x, vcache, tb + ML_TS, w, lane, vr);
  }

  // ---- sums over lanes and waves (every wave shares the same running max)
#pragma unroll
  for (int hb = 0; hb < NHB; ++hb) {
    float s = lsum[hb];
    s = rows4_sum(s);
    if (g == 0) wsum[w][16 * hb + c16] = s;
  }
  __syncthreads();   // also: every wave is done with Q, P and its V tile
  float* ob = reinterpret_cast<float*>(lds) + w * 32 * ML_OB_PITCH;   // [head][dim] of this wave's 64 dims
#pragma unroll
  for (int db = 0; db < ML_DW / 16; ++db)
#pragma unroll
    for (int hb = 0; hb < NHB; ++hb)
#pragma unroll
      for (int i = 0; i < 4; ++i) ob[(16 * hb + c16) * ML_OB_PITCH + 16 * db + 4 * g + i] = o[db][hb][i];
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  float* pml = a.part_ml + (size_t(unit) * a.splits + split) * G * 2;
  float* po = a.part_o + (size_t(unit) * a.splits + split) * G * ML_DV;
  const bool single = a.splits == 1;
  const size_t row0 = size_t(b) * a.Hq + size_t(kvh) * G;
  // 32 heads x 64 dims of this wave: 16 float4 per head row, 512 float4 per wave
  for (int idx = lane; idx < 16 * NHB * 16; idx += 64) {
    const int hl = idx >> 4, d4 = idx & 15, h = h0 + hl;
    if (h < G) {
      const float* src = ob + hl * ML_OB_PITCH + 4 * d4;
      float4 v = make_float4(src[0], src[1], src[2], src[3]);
      if (single) {
        float L = 0.f;
#pragma unroll
        for (int ww = 0; ww < ML_WAVES; ++ww) L += wsum[ww][hl];
        const float inv = L > 0.f ? 1.f / L : 0.f;
        v = make_float4(v.x * inv, v.y * inv, v.z * inv, v.w * inv);
        *reinterpret_cast<float4*>(a.out + (row0 + h) * ML_DV + ML_DW * w + 4 * d4) = v;
      } else {
        float* dst = po + size_t(h) * ML_DV + ML_DW * w + 4 * d4;
        if (a.fused) {
          st_dev(dst, v.x);
          st_dev(dst + 1, v.y);
          st_dev(dst + 2, v.z);
          st_dev(dst + 3, v.w);
        } else {
          *reinterpret_cast<float4*>(dst) = v;
        }
      }
    }
  }
  if (w == 0 && lane < 16 * NHB) {
    const int h = h0 + lane;
    if (h < G) {
      float L = 0.f;
#pragma unroll
      for (int ww = 0; ww < ML_WAVES; ++ww) L += wsum[ww][lane];
      const float M = (lane >> 4) ? m2[NHB - 1] : m2[0];   // lanes 0..15: head block 0, 16..31: block 1
      const float Mn = (M == -INFINITY) ? -INFINITY : M * 0.6931471805599453f;
      if (single) {
        if (a.lse != nullptr) a.lse[row0 + h] = L > 0.f ? Mn + logf(L) : -INFINITY;
      } else {
        st_part(a, pml + 2 * h, Mn);
        st_part(a, pml + 2 * h + 1, L);
      }
    }
  }
  if (a.fused) {
    int* ctr = a.counters + unit * ATTN_MAX_HG + hg;
    if (attn_split_done(ctr, a.splits)) attn_merge_splits<ML_THREADS>(a, unit, h0, min(32, G - h0), ctr);
  }
}

// ---------------------------------------------------------------------------
// Groups of 17..32 heads: 64-slot tiles with the next tile's rows in flight.
//
// Wave w = 4 ch + sg loads the rows of slots 16 sg .. 16 sg + 15 of a tile,
// columns 288 ch .. 288 ch + 287 (nine 32-column k-steps), into one of two
// register buffers: while a tile is scored and multiplied, the next tile's rows
// are already being fetched.  The two waves of a slot group each form partial
// scores over their column half for all 32 heads and swap the head block the
// other one owns through LDS, so wave (sg, ch) ends with the full scores of its
// 16 slots for heads 16 ch .. 16 ch + 15 and makes their P.  The rows' first
// 512 columns (the values) go from the same registers into a row-major LDS
// tile, which the P.V product reads with the gfx950 transposing LDS read
// (ds_read_b64_tr_b16): each row is fetched from HBM once and never re-read.
// Wave w owns output dims 64 w .. 64 w + 63 for all heads.
constexpr int MP_TS = 64;                                   // slots per tile
constexpr int MP_KH = ML_NKS / 2;                           // k-steps per column half (9)
constexpr int MP_VP = ML_DV + 16;                           // u16 per LDS value row (8-word bank skew)
constexpr int MP_V_BYTES = MP_TS * MP_VP * 2;               // 67584
constexpr int MP_P_BYTES = 2 * 2 * 2 * 2 * 64 * 8;          // 8192: [kstep][half][hb][hi/lo][lane] uint2
constexpr int MP_X_BYTES = 4 * 2 * 64 * 16;                 // 8192: [sg][hb][lane] partial scores
constexpr int MP_MAIN_BYTES = ML_Q_BYTES + MP_V_BYTES + MP_P_BYTES + MP_X_BYTES;
constexpr int MP_LDS_BYTES = MP_MAIN_BYTES > ML_OB_BYTES ? MP_MAIN_BYTES : ML_OB_BYTES;

typedef __attribute__((__vector_size__(4 * sizeof(__bf16)))) __bf16 mp_bf16x4;

// Transposing LDS read: within each 16-lane group, lane 4e + c supplies the address
// of 4 consecutive u16 (row e of a 4 x 16 block, columns 4c .. 4c + 3) and lane i
// receives column i of the block, rows 0..3.
__device__ __forceinline__ uint2 mp_read_tr(const uint16_t* p) {
  typedef __attribute__((address_space(3))) mp_bf16x4* lds_p;
  const mp_bf16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_p)(const __attribute__((address_space(3))) void*)p);
  uint2 r;
  __builtin_memcpy(&r, &v, 8);
  return r;
}

// This wave's rows (slot 16 sg + (lane & 15)) and column half: lane holds columns
// 288 ch + 32 c + 8 (lane >> 4) .. + 7 of k-step c.
__device__ __forceinline__ int mp_load(const MlCtx& x, const int32_t* vcache, int tb, int sg, int ch, int lane,
                                       u32x4 (&k)[MP_KH]) {
  const int tk = ml_token(x, vcache, tb + 16 * sg + (lane & 15));
  // unconditional loads keep the wait counts exact; a slot without a token reads row 0
  const uint32_t r = uint32_t(max(tk, 0)) * ML_DK + 288 * ch + 8 * (lane >> 4);
#pragma unroll
  for (int c = 0; c < MP_KH; ++c) k[c] = ld16(x.cu + r + 32 * c);
  return tk;
}

template <int SEL>
__global__ __launch_bounds__(ML_THREADS) void attn_mla_pf_kernel(AttnArgs a) {
  __shared__ __align__(16) unsigned char lds[MP_LDS_BYTES];
  __shared__ float wmax[4][32];
  __shared__ float wsum[4][32];
  __shared__ int32_t vcache[ML_VCACHE];
  const u32x4* qs = reinterpret_cast<const u32x4*>(lds);                                  // [NKS][hb][lane]
  uint16_t* vl = reinterpret_cast<uint16_t*>(lds + ML_Q_BYTES);                           // [slot][MP_VP]
  uint2* ps = reinterpret_cast<uint2*>(lds + ML_Q_BYTES + MP_V_BYTES);                    // [j][half][hb][hl][lane]
  f32x4* xs = reinterpret_cast<f32x4*>(lds + ML_Q_BYTES + MP_V_BYTES + MP_P_BYTES);      // [sg][hb][lane]
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int g = lane >> 4, c16 = lane & 15;
  const int sg = w & 3, ch = w >> 2;

  const int unit = blockIdx.y, split = blockIdx.x, hg = blockIdx.z;
  const int b = unit / a.Hkv, kvh = unit % a.Hkv;
  const int G = a.G, h0 = 32 * hg;
  const bool identity = SEL == 0 && a.view_idx == nullptr;
  // in-launch selection: the unit's page scores, loaded first (their addresses depend
  // on kernel arguments alone), masked by the page count once the length is known
  float sraw[SEL > 0 ? SEL : 1];
  if constexpr (SEL > 0) {
    const float* srow = a.sel_score + size_t(unit) * a.sel_ncp;
#pragma unroll
    for (int j = 0; j < SEL; ++j) sraw[j] = srow[min(topk_reg_index<ML_THREADS, SEL>(j), a.sel_ncp - 1)];
  }
  const int len0 = min(a.seq_len[b], a.cap);
  const int len = (SEL > 0 && len0 < a.cap) ? len0 + 1 : len0;   // the row the scoring launch appended
  const int n_slots = identity ? len : a.view_cap * a.gran;
  const int s_valid = identity ? len : (SEL > 0 ? 0 : min(a.view_len[unit], a.view_cap) * a.gran);
  int chunk = (n_slots + a.splits - 1) / a.splits;
  chunk = (chunk + MP_TS - 1) / MP_TS * MP_TS;
  const int s0 = min(n_slots, split * chunk), s1 = min(n_slots, s0 + chunk);
  const int ntiles = (s1 - s0 + MP_TS - 1) / MP_TS;

  MlCtx x;
  x.cu = (const uint16_t*)a.k + size_t(unit) * a.cap * ML_DK;
  x.len = len;
  x.s1 = min(s1, s_valid);
  x.gshift = a.gshift;
  x.identity = identity;
  x.e0 = 0;
  // Q (in B-operand order: entry (c, hb, lane) = head h0 + 16 hb + (lane & 15), columns
  // 32c + 8(lane >> 4) .. + 7) and the view entries of this split are fetched together
  constexpr int QN = ML_NKS * 2 * 64, QR = (QN + ML_THREADS - 1) / ML_THREADS;
  u32x4 qv[QR];
#pragma unroll
  for (int r = 0; r < QR; ++r) {
    const int i = threadIdx.x + r * ML_THREADS;
    const int l = i & 63, hb = (i >> 6) & 1, c = i >> 7;
    const int h = h0 + 16 * hb + (l & 15);
    // unconditional loads (clamped in range, zeroed after) keep the wait counts exact
    const int hc = min(h, G - 1), cc = min(c, ML_NKS - 1);
    qv[r] = ld16((const uint16_t*)a.q + (size_t(b) * a.Hq + size_t(kvh) * G + hc) * ML_DK + 32 * cc + 8 * (l >> 4));
    if (!(i < QN && h < G)) qv[r] = u32x4{0u, 0u, 0u, 0u};
  }
  // at most ML_VCACHE - 1 entries (attn_mla_supported)
  constexpr int VR = ML_VCACHE / ML_THREADS;
  int32_t ve[VR];
  int e0 = 0, e1 = 0;
  if (!identity && SEL == 0) {
    const int32_t* vrow = a.view_idx + size_t(unit) * a.view_cap;
    e0 = s0 >> a.gshift;
    e1 = s1 > s0 ? ((s1 - 1) >> a.gshift) + 1 : e0;
#pragma unroll
    for (int r = 0; r < VR; ++r) {
      const int e = e0 + threadIdx.x + r * ML_THREADS;
      ve[r] = e < e1 ? vrow[e] : -1;
    }
    x.e0 = e0;
  }
  auto stage_q = [&]() {
#pragma unroll
    for (int r = 0; r < QR; ++r) {
      const int i = threadIdx.x + r * ML_THREADS;
      if (i < QN) reinterpret_cast<u32x4*>(lds)[i] = qv[r];
    }
  };
  if constexpr (SEL == 0) stage_q();
  if (!identity && SEL == 0) {
#pragma unroll
    for (int r = 0; r < VR; ++r) {
      const int e = e0 + threadIdx.x + r * ML_THREADS;
      if (e < e1) vcache[e - e0] = ve[r];
    }
  }
  int sel_len = 0;
  if constexpr (SEL > 0) {
    // the unit's top pages by score, ascending, straight into the view cache (the
    // value tile is not in use yet and holds the selection's histograms)
    using SelShared = TopkRegSharedN<ML_WAVES, 2>;
    static_assert(sizeof(SelShared) <= MP_V_BYTES, "selection scratch");
    SelShared& tsh = *reinterpret_cast<SelShared*>(lds + ML_Q_BYTES);
    const int npages = min((len + a.gran - 1) >> a.gshift, a.sel_ncp);
    uint32_t key[SEL > 0 ? SEL : 1];
#pragma unroll
    for (int j = 0; j < SEL; ++j) key[j] = topk_reg_index<ML_THREADS, SEL>(j) < npages ? ordered_bits(sraw[j]) : 0u;
    sel_len = block_topk_keys<ML_THREADS, SEL, SelShared>(key, npages, a.view_cap, vcache, tsh);
    stage_q();   // after the selection: q's loads return while it runs
  }
  __syncthreads();
  if constexpr (SEL > 0) {
    x.s1 = min(s1, min(sel_len, a.view_cap) * a.gran);
    if (split == 0 && hg == 0 && a.sel_view != nullptr) {
      for (int i = threadIdx.x; i < a.view_cap; i += ML_THREADS) a.sel_view[size_t(unit) * a.view_cap + i] = vcache[i];
      if (threadIdx.x == 0) a.sel_vlen[unit] = sel_len;
    }
  }
  u32x4 kb0[MP_KH], kb1[MP_KH];
  // unconditional (slots past the split read row 0): the loop's wait counts stay exact
  int tk0 = mp_load(x, vcache, s0, sg, ch, lane, kb0), tk1 = -1;

  const float sc2 = a.scale * LOG2E;
  f32x4 o[ML_DW / 16][2];
#pragma unroll
  for (int db = 0; db < ML_DW / 16; ++db) o[db][0] = o[db][1] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m2[2] = {-INFINITY, -INFINITY};
  float lsum = 0.f;                  // head 16 ch + c16, this wave's slots
  // transposing-read source row / column of this lane (see mp_read_tr)
  const int tr_row = 4 * g + ((lane >> 2) & 3), tr_col = ML_DW * w + 4 * (lane & 3);

  auto step = [&](u32x4 (&cur)[MP_KH], int& tkc, u32x4 (&nxt)[MP_KH], int& tkn, int it, auto pref) {
    const int tb = s0 + it * MP_TS;
    if constexpr (decltype(pref)::value) {
      tkn = mp_load(x, vcache, tb + MP_TS, sg, ch, lane, nxt);
    }
    // ---- partial scores over this wave's column half, both head blocks
    f32x4 sa0 = {0.f, 0.f, 0.f, 0.f}, sa1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int c = 0; c < MP_KH; ++c) {
      sa0 = mfma_bf16_16x16x32(cur[c], qs[((MP_KH * ch + c) * 2 + 0) * 64 + lane], sa0);
      sa1 = mfma_bf16_16x16x32(cur[c], qs[((MP_KH * ch + c) * 2 + 1) * 64 + lane], sa1);
    }
    xs[(sg * 2 + (1 - ch)) * 64 + lane] = ch ? sa0 : sa1;   // the partner's head block
    __syncthreads();
    const f32x4 oth = xs[(sg * 2 + ch) * 64 + lane];
    const f32x4 own = ch ? sa1 : sa0;
    // value columns of these rows into the LDS tile (rope columns 512.. stay out)
    uint16_t* vdst = vl + (16 * sg + c16) * MP_VP + 288 * ch + 8 * g;
#pragma unroll
    for (int c = 0; c < MP_KH; ++c)
      if (ch == 0 || c < 7) *reinterpret_cast<u32x4*>(vdst + 32 * c) = cur[c];
    const uint64_t valid = __ballot(tkc >= 0);
    float sv[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) sv[i] = ((valid >> (4 * g + i)) & 1) ? (own[i] + oth[i]) * sc2 : -INFINITY;
    if (a.logits != nullptr) {
      const int h = h0 + 16 * ch + c16;
      if (h < G) {
        float* row = a.logits + (size_t(b) * a.Hq + size_t(kvh) * G + h) * a.logit_cap;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int s = tb + 16 * sg + 4 * g + i;
          if (s < x.s1 && s < a.logit_cap)
            row[s] = ((valid >> (4 * g + i)) & 1) ? (own[i] + oth[i]) * a.scale : -INFINITY;
        }
      }
    }
    {
      float m = fmaxf(fmaxf(sv[0], sv[1]), fmaxf(sv[2], sv[3]));
      m = rows4_max(m);
      if (g == 0) wmax[sg][16 * ch + c16] = m;
    }
    __syncthreads();
    // ---- tile maxima of both head blocks; every wave takes the same decisions
#pragma unroll
    for (int hb = 0; hb < 2; ++hb) {
      const float tmax = fmaxf(fmaxf(wmax[0][16 * hb + c16], wmax[1][16 * hb + c16]),
                               fmaxf(wmax[2][16 * hb + c16], wmax[3][16 * hb + c16]));
      const bool grow = tmax > m2[hb] + ML_MARGIN;
      if (__ballot(grow) != 0) {
        const float mnew = grow ? tmax : m2[hb];
        const float alpha = (grow && m2[hb] != -INFINITY) ? ex2(m2[hb] - mnew) : 1.f;
        if (hb == ch) lsum *= alpha;
#pragma unroll
        for (int db = 0; db < ML_DW / 16; ++db) o[db][hb] *= alpha;
        m2[hb] = mnew;
      }
    }
    {
      const float mo = ch ? m2[1] : m2[0];
      const float mref = mo == -INFINITY ? 0.f : mo;
      float p[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        p[i] = ex2(sv[i] - mref);   // 0 for masked slots, at most 2^8 otherwise
        lsum += p[i];
      }
      uint2 hi, lo;
      hi.x = pack_bf16(p[0], p[1]);
      hi.y = pack_bf16(p[2], p[3]);
      lo.x = pack_bf16(p[0] - bf16x2_lo_f32(hi.x), p[1] - bf16x2_hi_f32(hi.x));
      lo.y = pack_bf16(p[2] - bf16x2_lo_f32(hi.y), p[3] - bf16x2_hi_f32(hi.y));
      // slots 16 sg + 4g + i: k-step sg >> 1, half sg & 1
      ps[((((sg >> 1) * 2 + (sg & 1)) * 2 + ch) * 2 + 0) * 64 + lane] = hi;
      ps[((((sg >> 1) * 2 + (sg & 1)) * 2 + ch) * 2 + 1) * 64 + lane] = lo;
    }
    __syncthreads();
    // ---- O^T += V^T P^T over the tile's two 32-slot k-steps.  Both operands take the
    // k order (4a .. 4a + 3, 16 + 4a .. 16 + 4a + 3) for lane group a.
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      u32x4 ph[2], pl[2];
#pragma unroll
      for (int hb = 0; hb < 2; ++hb) {
        const uint2 h0v = ps[(((j * 2 + 0) * 2 + hb) * 2 + 0) * 64 + lane];
        const uint2 h1v = ps[(((j * 2 + 1) * 2 + hb) * 2 + 0) * 64 + lane];
        const uint2 l0v = ps[(((j * 2 + 0) * 2 + hb) * 2 + 1) * 64 + lane];
        const uint2 l1v = ps[(((j * 2 + 1) * 2 + hb) * 2 + 1) * 64 + lane];
        ph[hb] = u32x4{h0v.x, h0v.y, h1v.x, h1v.y};
        pl[hb] = u32x4{l0v.x, l0v.y, l1v.x, l1v.y};
      }
#pragma unroll
      for (int db = 0; db < ML_DW / 16; ++db) {
        const uint16_t* src = vl + (32 * j + tr_row) * MP_VP + tr_col + 16 * db;
        const uint2 x0 = mp_read_tr(src), x1 = mp_read_tr(src + 16 * MP_VP);
        const u32x4 av = {x0.x, x0.y, x1.x, x1.y};
#pragma unroll
        for (int hb = 0; hb < 2; ++hb) {
          o[db][hb] = mfma_bf16_16x16x32(av, ph[hb], o[db][hb]);
          o[db][hb] = mfma_bf16_16x16x32(av, pl[hb], o[db][hb]);
        }
      }
    }
  };
  using Pf = std::integral_constant<bool, true>;
  using NoPf = std::integral_constant<bool, false>;
  int it = 0;
  for (; it + 2 < ntiles; it += 2) {
    step(kb0, tk0, kb1, tk1, it, Pf{});
    step(kb1, tk1, kb0, tk0, it + 1, Pf{});
  }
  if (ntiles - it == 2) {
    step(kb0, tk0, kb1, tk1, it, Pf{});
    step(kb1, tk1, kb0, tk0, it + 1, NoPf{});
  } else if (ntiles - it == 1) {
    step(kb0, tk0, kb1, tk1, it, NoPf{});
  }

  int row_ticket = 0;
  if (SEL > 0 && threadIdx.x == 0) {
    // every block of the batch row takes a ticket, long after it read the old length;
    // the last one stores the new length at the end
    row_ticket = __hip_atomic_fetch_add(a.row_ctr + b, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  // ---- sums over lanes and slot groups (every wave shares the same running max)
  {
    const float s = rows4_sum(lsum);
    if (g == 0) wsum[sg][16 * ch + c16] = s;
  }
  __syncthreads();   // also: every wave is done with Q, P and the value tile
  float* ob = reinterpret_cast<float*>(lds) + w * 32 * ML_OB_PITCH;   // [head][dim] of this wave's 64 dims
#pragma unroll
  for (int db = 0; db < ML_DW / 16; ++db)
#pragma unroll
    for (int hb = 0; hb < 2; ++hb)
#pragma unroll
      for (int i = 0; i < 4; ++i) ob[(16 * hb + c16) * ML_OB_PITCH + 16 * db + 4 * g + i] = o[db][hb][i];
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  float* pml = a.part_ml + (size_t(unit) * a.splits + split) * G * 2;
  float* po = a.part_o + (size_t(unit) * a.splits + split) * G * ML_DV;
  const bool single = a.splits == 1;
  const size_t row0 = size_t(b) * a.Hq + size_t(kvh) * G;
  // 32 heads x 64 dims of this wave: 16 float4 per head row, 512 float4 per wave
  for (int idx = lane; idx < 32 * 16; idx += 64) {
    const int hl = idx >> 4, d4 = idx & 15, h = h0 + hl;
    if (h < G) {
      const float* src = ob + hl * ML_OB_PITCH + 4 * d4;
      float4 v = make_float4(src[0], src[1], src[2], src[3]);
      if (single) {
        const float L = (wsum[0][hl] + wsum[1][hl]) + (wsum[2][hl] + wsum[3][hl]);
        const float inv = L > 0.f ? 1.f / L : 0.f;
        v = make_float4(v.x * inv, v.y * inv, v.z * inv, v.w * inv);
        *reinterpret_cast<float4*>(a.out + (row0 + h) * ML_DV + ML_DW * w + 4 * d4) = v;
      } else {
        float* dst = po + size_t(h) * ML_DV + ML_DW * w + 4 * d4;
        if (a.fused) {
          st_dev(dst, v.x);
          st_dev(dst + 1, v.y);
          st_dev(dst + 2, v.z);
          st_dev(dst + 3, v.w);
        } else {
          *reinterpret_cast<float4*>(dst) = v;
        }
      }
    }
  }
  if (w == 0 && lane < 32) {
    const int h = h0 + lane;
    if (h < G) {
      const float L = (wsum[0][lane] + wsum[1][lane]) + (wsum[2][lane] + wsum[3][lane]);
      const float M = (lane >> 4) ? m2[1] : m2[0];
      const float Mn = (M == -INFINITY) ? -INFINITY : M * 0.6931471805599453f;
      if (single) {
        if (a.lse != nullptr) a.lse[row0 + h] = L > 0.f ? Mn + logf(L) : -INFINITY;
      } else {
        st_part(a, pml + 2 * h, Mn);
        st_part(a, pml + 2 * h + 1, L);
      }
    }
  }
  if (a.fused) {
    int* ctr = a.counters + unit * ATTN_MAX_HG + hg;
    if (attn_split_done(ctr, a.splits)) attn_merge_splits<ML_THREADS>(a, unit, h0, min(32, G - h0), ctr);
  }
  if (SEL > 0 && threadIdx.x == 0 && row_ticket == a.Hkv * a.splits * int(gridDim.z) - 1) {   // all have read it
    if (len != len0) a.seq_len_w[b] = len;
    ticket_reset(a.row_ctr + b);
  }
}

// Keys per thread of the in-launch page selection for sel_ncp pages (0: too many).
int attn_mla_sel_keys(int ncp) {
  return ncp <= ML_THREADS * 4 ? 4 : ncp <= ML_THREADS * 8 ? 8 : ncp <= ML_THREADS * 16 ? 16 : 0;
}

bool attn_mla_supported(const AttnArgs& a) {
  if (!(a.dtype == SE_BF16 && a.latent && a.Dk == ML_DK && a.Dv == ML_DV && a.G <= 64)) return false;
  if (a.cap > (1 << 30) / ML_DK) return false;
  if (a.view_idx != nullptr) {
    if (a.gshift < 0) return false;
    const int slots = a.view_cap * a.gran;
    int chunk = (slots + a.splits - 1) / a.splits;
    chunk = (chunk + ML_TS - 1) / ML_TS * ML_TS;
    if (chunk / a.gran + 2 > ML_VCACHE) return false;
  }
  return true;
}

// One block per CU when the units alone do not fill the chip.
int attn_mla_auto_splits(int units, int G, int slots) {
  const int blocks_per_split = units * ((G + 31) / 32);
  int s = (256 + blocks_per_split - 1) / blocks_per_split;
  s = std::max(1, std::min(s, (slots + ML_TS - 1) / ML_TS));
  return std::min(s, 256);
}

se_status launch_attn_mla(const AttnArgs& a, hipStream_t s) {
  dim3 grid(a.splits, a.B * a.Hkv, (a.G + 31) / 32);
  if (a.sel) {   // the fused decode step: groups of 17..32 heads, a view that fits the view cache
    const int e = attn_mla_sel_keys(a.sel_ncp);
    if (a.G <= 16 || a.G > 32 || a.view_cap > ML_VCACHE || a.gshift < 0 || e == 0) return SE_ERR_UNSUPPORTED;
    if (e == 4) hipLaunchKernelGGL((attn_mla_pf_kernel<4>), grid, dim3(ML_THREADS), 0, s, a);
    else if (e == 8) hipLaunchKernelGGL((attn_mla_pf_kernel<8>), grid, dim3(ML_THREADS), 0, s, a);
    else hipLaunchKernelGGL((attn_mla_pf_kernel<16>), grid, dim3(ML_THREADS), 0, s, a);
  } else if (a.G <= 16) {
    hipLaunchKernelGGL((attn_mla_kernel<1>), grid, dim3(ML_THREADS), 0, s, a);
  } else {
    hipLaunchKernelGGL((attn_mla_pf_kernel<0>), grid, dim3(ML_THREADS), 0, s, a);
  }
  return launch_status();
}

}  // namespace se
