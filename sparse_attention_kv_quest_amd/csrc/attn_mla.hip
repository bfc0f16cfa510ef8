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
// Block: 8 waves, one (unit, split, group of 32 heads); tiles of 128 view
// slots.  Wave w scores slots 16w..16w+15 of a tile over all 576 columns (K
// rows go from HBM straight into A-operand registers; Q is staged once in LDS
// in B-operand order), and owns output dims 64w..64w+63 for all heads: it
// loads those 64 columns of all 128 rows a second time in a four-token-per-
// lane order (an L2 hit), which a v_perm transpose turns into V^T in a
// wave-private LDS tile.  Softmax state is shared through LDS: the waves post
// their per-head maxima, all of them take the same tile maximum and make the
// same (lazy, 2^8-margin) rescaling decision, and each wave posts P of its own
// slots as bf16 hi + lo pairs that every wave then reads as the B operand.
// The next tile's K loads are issued as soon as the scores are formed and its
// V loads as soon as the transposes are done, so a tile of rows is always in
// flight.  Each split stores a partial (max, sum, output), which the combine
// kernel merges (or, for small partials, the block finishing the last split).
#include "attn_common.hpp"
#include "mfma_util.hpp"

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
    const int page = s < x.s1 ? vcache[(s >> x.gshift) - x.e0] : -1;
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
  if (a.G <= 16)
    hipLaunchKernelGGL((attn_mla_kernel<1>), grid, dim3(ML_THREADS), 0, s, a);
  else
    hipLaunchKernelGGL((attn_mla_kernel<2>), grid, dim3(ML_THREADS), 0, s, a);
  return launch_status();
}

}  // namespace se
