// Grouped-query causal prefill attention for gfx950 (MI355X) with the fused
// QK-norm + RoPE prologue on every query and key row.
//
// Algorithm (the pages):
//  * "ADR-0060: AHBM GQA Fused Attention Kernel (Llama3-70B)", section 3:
//    tiled online softmax (FlashAttention) over K/V tiles; section 5.4: a
//    key tile entirely in the future of a query block is skipped, one
//    entirely in its past needs no mask, an overlapping one gets the
//    triangular mask; section 5.2: query head h reads KV head floor(h / G).
//  * "Qwen3-14B Optimization", section 2.1 "Shape 4" / #796: QK-norm and
//    RoPE are applied inside the attention stage; #602: RoPE on lo/hi halves.
//
// gfx950 mapping:
//  * one workgroup = (128-query tile, query head, sequence), 4 waves of 32
//    query rows, on a 1-D grid ordered so that all workgroups of one KV head
//    land on one XCD (shared L2), heaviest (last) query tile first.
//  * per 64-key tile: raw K/V rows are fetched into registers one tile ahead,
//    the key prologue runs on them (f32), K' (bf16) and V go to LDS;
//    S^T = K' Q'^T and O^T = V^T P^T run on v_mfma_f32_32x32x16_bf16 with
//    f32 accumulation.  In the S^T orientation a lane owns one query row, so
//    the row max needs one cross-lane step.  K' rows are XOR-swizzled in
//    16-byte chunks so the MFMA operand reads are bank-conflict free.
//  * scores live in the log2 domain (scale * log2 e folded in) and use the
//    hardware exp2.
#include "common.hpp"

namespace gqa {
namespace {

constexpr int kWaves = 4;
constexpr int kThreads = 256;
constexpr int BM = kPrefillBM;   // 128
constexpr int BN = kPrefillBN;   // 64
constexpr int kXcds = 8;         // MI355X: 8 accelerator complex dies, each with its own L2

struct __attribute__((aligned(16))) PrefillSmem {
  uint32_t kt[BN][kHeadDim / 2];   // K' tile, bf16 pairs, 16-byte chunks swizzled by key & 15
  uint32_t vt[BN][kHeadDim / 2];   // V tile, bf16 pairs, row-major
  double inv_rev[kHeadDim / 2];    // theta^(-2i/128) / (2 pi)
  float gk[kHeadDim];              // key RMSNorm weight (f32)
};

// Logical 16-byte chunk (of 16 per 128-dim row) holding operand slot kk of
// lane half hf: the lane's 8 slots cover dims [32hf, 32hf+32) and
// [64+32hf, 64+32hf+32), so every RoPE pair (i, i+64) stays in one lane.
__device__ __forceinline__ int qk_chunk(int kk, int hf) { return kk < 4 ? 4 * hf + kk : 8 + 4 * hf + (kk - 4); }

__global__ __launch_bounds__(kThreads, 2) void prefill_kernel(const PrefillParams p) {
  __shared__ PrefillSmem sm;

  // XCD-aware workgroup order: consecutive workgroup ids are dealt round-robin
  // to the 8 XCDs, so when the (sequence, KV head) groups divide evenly every
  // group's workgroups share one XCD and its K/V tiles stay in that XCD's L2.
  // Within a group: heaviest (last) query tile first, the G query heads of a
  // tile adjacent.
  const int G = p.group;
  const int per_group = p.n_qtiles * G;
  const int groups = p.batch * p.num_kv_heads;
  const int bid = blockIdx.x;
  int grp, w;
  if (groups % kXcds == 0) {
    const int slot = bid / kXcds;
    grp = bid % kXcds + kXcds * (slot / per_group);
    w = slot % per_group;
  } else {
    grp = bid / per_group;
    w = bid % per_group;
  }
  const int b = grp / p.num_kv_heads, h = grp % p.num_kv_heads;
  const int qt = p.n_qtiles - 1 - w / G;
  const int hq = h * G + w % G;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int n32 = lane & 31, hf = lane >> 5;

  int n = p.seq_lens[b];
  n = n < 0 ? 0 : (n > p.max_seq ? p.max_seq : n);
  const int qs = qt * BM;
  if (qs >= n) return;
  const int qe = min(qs + BM, n);
  const int kend = p.causal ? qe : n;            // keys [0, kend) can be visible
  const int ntiles = (kend + BN - 1) / BN;
  const bool rope = p.rope_theta > 0.0;
  const double pos0 = (double)p.positions[b];

  // ---- tables: RoPE inverse frequencies (revolutions) and key norm weight
  if (tid < 64 && rope) sm.inv_rev[tid] = pow(p.rope_theta, -2.0 * (double)tid / (double)kHeadDim) * 0.15915494309189535;
  if (tid < kHeadDim) sm.gk[tid] = p.k_norm_w ? bf16lo(((const uint16_t*)p.k_norm_w)[tid]) : 1.0f;
  __syncthreads();

  // ---- query prologue: lane (n32, hf) owns row qs + 32*wave + n32, dims
  //      [32hf, 32hf+32) and [64+32hf, 64+32hf+32)
  const int qrow = qs + 32 * wave + n32;
  bf16x8 qf[8];
  {
    float xl[32], xh[32];
    if (qrow < n) {
      const uint16_t* row = (const uint16_t*)p.q + ((int64_t)b * p.q_sb + (int64_t)hq * p.q_sh + (int64_t)qrow * p.q_ss);
      #pragma unroll
      for (int j = 0; j < 4; ++j) {
        const u32x4 lo = *(const u32x4*)(row + 32 * hf + 8 * j);
        const u32x4 hi = *(const u32x4*)(row + 64 + 32 * hf + 8 * j);
        #pragma unroll
        for (int e = 0; e < 8; ++e) {
          xl[8 * j + e] = bf16_elem(lo, e);
          xh[8 * j + e] = bf16_elem(hi, e);
        }
      }
    } else {
      #pragma unroll
      for (int e = 0; e < 32; ++e) xl[e] = xh[e] = 0.f;
    }
    if (p.q_norm_w) {
      float ss = 0.f;
      #pragma unroll
      for (int e = 0; e < 32; ++e) ss += xl[e] * xl[e] + xh[e] * xh[e];
      ss += __shfl_xor(ss, 32, 64);
      const float r = 1.0f / sqrtf(ss * (1.0f / kHeadDim) + p.eps);
      const uint16_t* g = (const uint16_t*)p.q_norm_w;
      #pragma unroll
      for (int e = 0; e < 32; ++e) {
        xl[e] *= r * bf16lo(g[32 * hf + e]);
        xh[e] *= r * bf16lo(g[64 + 32 * hf + e]);
      }
    }
    if (rope) {
      const double qpos = pos0 + (double)qrow;
      #pragma unroll
      for (int e = 0; e < 32; ++e) {
        float c, s;
        rope_cos_sin_rev(qpos, sm.inv_rev[32 * hf + e], c, s);
        const float lo = xl[e], hi = xh[e];
        xl[e] = lo * c - hi * s;
        xh[e] = hi * c + lo * s;
      }
    }
    #pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      qf[kk] = as_bf16x8(u32x4{pack_bf16x2(xl[8 * kk], xl[8 * kk + 1]), pack_bf16x2(xl[8 * kk + 2], xl[8 * kk + 3]),
                               pack_bf16x2(xl[8 * kk + 4], xl[8 * kk + 5]), pack_bf16x2(xl[8 * kk + 6], xl[8 * kk + 7])});
      qf[4 + kk] = as_bf16x8(u32x4{pack_bf16x2(xh[8 * kk], xh[8 * kk + 1]), pack_bf16x2(xh[8 * kk + 2], xh[8 * kk + 3]),
                                   pack_bf16x2(xh[8 * kk + 4], xh[8 * kk + 5]), pack_bf16x2(xh[8 * kk + 6], xh[8 * kk + 7])});
    }
  }

  // ---- per-thread K/V tile loading roles
  const int lkey = tid >> 2, part = tid & 3;     // key prologue: 16 pairs (i, i+64), i in [16 part, 16 part + 16)
  const uint16_t* kslab = (const uint16_t*)p.k + ((int64_t)b * p.k_sb + (int64_t)h * p.k_sh);
  const uint16_t* vslab = (const uint16_t*)p.v + ((int64_t)b * p.v_sb + (int64_t)h * p.v_sh);
  struct Raw { u32x4 k0, k1, k2, k3, v0, v1, v2, v3; } raw;
#define GQA_FETCH_TILE(KT)                                                       \
  do {                                                                           \
    const int key_ = (KT) * BN + lkey;                                           \
    if (key_ < n) {                                                              \
      const uint16_t* kr_ = kslab + (int64_t)key_ * p.k_ss + 16 * part;         \
      const uint16_t* vr_ = vslab + (int64_t)key_ * p.v_ss + 32 * part;         \
      raw.k0 = *(const u32x4*)(kr_);                                             \
      raw.k1 = *(const u32x4*)(kr_ + 8);                                         \
      raw.k2 = *(const u32x4*)(kr_ + 64);                                        \
      raw.k3 = *(const u32x4*)(kr_ + 72);                                        \
      raw.v0 = *(const u32x4*)(vr_);                                             \
      raw.v1 = *(const u32x4*)(vr_ + 8);                                         \
      raw.v2 = *(const u32x4*)(vr_ + 16);                                        \
      raw.v3 = *(const u32x4*)(vr_ + 24);                                        \
    } else {                                                                     \
      raw.k0 = raw.k1 = raw.k2 = raw.k3 = u32x4{0, 0, 0, 0};                     \
      raw.v0 = raw.v1 = raw.v2 = raw.v3 = u32x4{0, 0, 0, 0};                     \
    }                                                                            \
  } while (0)

  f32x16 o[4];
  #pragma unroll
  for (int T = 0; T < 4; ++T)
    #pragma unroll
    for (int i = 0; i < 16; ++i) o[T][i] = 0.f;
  float m_run = -INFINITY, l_run = 0.f;
  const int wq0 = qs + 32 * wave;                 // this wave's first query
  const bool wave_live = wq0 < n;

  GQA_FETCH_TILE(0);
  for (int kt = 0; kt < ntiles; ++kt) {
    // ---- key prologue on the fetched rows -> K' (bf16) and V into LDS
    {
      float xl[16], xh[16];
      #pragma unroll
      for (int e = 0; e < 8; ++e) {
        xl[e] = bf16_elem(raw.k0, e);
        xl[8 + e] = bf16_elem(raw.k1, e);
        xh[e] = bf16_elem(raw.k2, e);
        xh[8 + e] = bf16_elem(raw.k3, e);
      }
      if (p.k_norm_w) {
        float ss = 0.f;
        #pragma unroll
        for (int e = 0; e < 16; ++e) ss += xl[e] * xl[e] + xh[e] * xh[e];
        ss += __shfl_xor(ss, 1, 4);
        ss += __shfl_xor(ss, 2, 4);
        const float r = 1.0f / sqrtf(ss * (1.0f / kHeadDim) + p.eps);
        #pragma unroll
        for (int e = 0; e < 16; ++e) {
          xl[e] *= r * sm.gk[16 * part + e];
          xh[e] *= r * sm.gk[64 + 16 * part + e];
        }
      }
      if (rope) {
        const double kpos = pos0 + (double)(kt * BN + lkey);
        #pragma unroll
        for (int e = 0; e < 16; ++e) {
          float c, s;
          rope_cos_sin_rev(kpos, sm.inv_rev[16 * part + e], c, s);
          const float lo = xl[e], hi = xh[e];
          xl[e] = lo * c - hi * s;
          xh[e] = hi * c + lo * s;
        }
      }
      const int sw = lkey & 15;
      uint32_t* krow = sm.kt[lkey];
      // logical chunks 2part, 2part+1 (lo half) and 8+2part, 9+2part (hi half)
      #pragma unroll
      for (int cc = 0; cc < 2; ++cc) {
        *(u32x4*)(krow + 4 * ((2 * part + cc) ^ sw)) =
            u32x4{pack_bf16x2(xl[8 * cc], xl[8 * cc + 1]), pack_bf16x2(xl[8 * cc + 2], xl[8 * cc + 3]),
                  pack_bf16x2(xl[8 * cc + 4], xl[8 * cc + 5]), pack_bf16x2(xl[8 * cc + 6], xl[8 * cc + 7])};
        *(u32x4*)(krow + 4 * ((8 + 2 * part + cc) ^ sw)) =
            u32x4{pack_bf16x2(xh[8 * cc], xh[8 * cc + 1]), pack_bf16x2(xh[8 * cc + 2], xh[8 * cc + 3]),
                  pack_bf16x2(xh[8 * cc + 4], xh[8 * cc + 5]), pack_bf16x2(xh[8 * cc + 6], xh[8 * cc + 7])};
      }
      uint32_t* vrow = sm.vt[lkey] + 16 * part;
      *(u32x4*)(vrow) = raw.v0;
      *(u32x4*)(vrow + 4) = raw.v1;
      *(u32x4*)(vrow + 8) = raw.v2;
      *(u32x4*)(vrow + 12) = raw.v3;
    }
    __syncthreads();
    if (kt + 1 < ntiles) GQA_FETCH_TILE(kt + 1);

    const int ks = kt * BN;
    // tile classification for this wave's 32 queries [wq0, wq0 + 32)
    const bool future = p.causal && ks > wq0 + 31;
    if (wave_live && !future) {
      const bool need_mask = (p.causal && ks + BN - 1 > wq0) || ks + BN > n;
      // S^T for two 32-key subtiles: sacc[u][i] = S[key ks + 32u + 8(i/4) + 4hf + i%4][query wq0 + n32]
      f32x16 sacc[2];
      #pragma unroll
      for (int u = 0; u < 2; ++u) {
        #pragma unroll
        for (int i = 0; i < 16; ++i) sacc[u][i] = 0.f;
        const int krow = 32 * u + n32;
        const uint32_t* kr = sm.kt[krow];
        const int sw = krow & 15;
        #pragma unroll
        for (int kk = 0; kk < 8; ++kk) {
          const u32x4 a = *(const u32x4*)(kr + 4 * (qk_chunk(kk, hf) ^ sw));
          sacc[u] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(a), qf[kk], sacc[u], 0, 0, 0);
        }
      }
      float mx = -INFINITY;
      #pragma unroll
      for (int u = 0; u < 2; ++u) {
        #pragma unroll
        for (int i = 0; i < 16; ++i) {
          float s = sacc[u][i] * p.scale_log2;
          if (need_mask) {
            const int key = ks + 32 * u + 8 * (i >> 2) + 4 * hf + (i & 3);
            if (key >= n || (p.causal && key > qrow)) s = -INFINITY;
          }
          sacc[u][i] = s;
          mx = fmaxf(mx, s);
        }
      }
      mx = wave_max_xor(mx, 32);
      const float m_new = fmaxf(m_run, mx);
      const float corr = fast_exp2(m_run - m_new);
      float ps = 0.f;
      #pragma unroll
      for (int u = 0; u < 2; ++u)
        #pragma unroll
        for (int i = 0; i < 16; ++i) {
          const float e = fast_exp2(sacc[u][i] - m_new);
          sacc[u][i] = e;
          ps += e;
        }
      l_run = l_run * corr + ps;
      m_run = m_new;
      #pragma unroll
      for (int T = 0; T < 4; ++T) o[T] *= corr;

      // O^T += V^T P^T: MFMA (u, e) takes keys ks + 32u + 16e + {4hf + t, 8 + 4hf + t}, t < 4
      #pragma unroll
      for (int u = 0; u < 2; ++u) {
        #pragma unroll
        for (int e = 0; e < 2; ++e) {
          const u32x4 pf = {pack_bf16x2(sacc[u][8 * e + 0], sacc[u][8 * e + 1]), pack_bf16x2(sacc[u][8 * e + 2], sacc[u][8 * e + 3]),
                            pack_bf16x2(sacc[u][8 * e + 4], sacc[u][8 * e + 5]), pack_bf16x2(sacc[u][8 * e + 6], sacc[u][8 * e + 7])};
          #pragma unroll
          for (int w = 0; w < 2; ++w) {          // dword w of each row: dims 4*n32 + 2w, 4*n32 + 2w + 1
            uint32_t r[8];
            #pragma unroll
            for (int t = 0; t < 8; ++t) {
              const int key = 32 * u + 16 * e + 4 * hf + (t < 4 ? t : 4 + t);
              r[t] = sm.vt[key][2 * n32 + w];
            }
            u32x4 a0, a1;
            #pragma unroll
            for (int uu = 0; uu < 4; ++uu) {
              a0[uu] = pair_lo(r[2 * uu], r[2 * uu + 1]);
              a1[uu] = pair_hi(r[2 * uu], r[2 * uu + 1]);
            }
            o[2 * w] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(a0), as_bf16x8(pf), o[2 * w], 0, 0, 0);
            o[2 * w + 1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(a1), as_bf16x8(pf), o[2 * w + 1], 0, 0, 0);
          }
        }
      }
    }
    __syncthreads();
  }

#undef GQA_FETCH_TILE

  // ---- epilogue: O / l for this lane's query row
  if (qrow >= n) return;
  l_run = wave_sum_xor(l_run, 32);
  const float inv = 1.0f / l_run;
  uint8_t* orow = (uint8_t*)p.out + ((int64_t)b * p.o_sb + (int64_t)hq * p.o_sh + (int64_t)qrow * p.o_ss) * (p.out_bf16 ? 2 : 4);
  // o[T][i] = O[query][dim 4*(8(i/4) + 4hf + i%4) + T]; per a = i/4 the 16 dims [32a + 16hf, 32a + 16hf + 16)
  #pragma unroll
  for (int a = 0; a < 4; ++a) {
    float v[16];
    #pragma unroll
    for (int r = 0; r < 4; ++r)
      #pragma unroll
      for (int T = 0; T < 4; ++T) v[4 * r + T] = o[T][4 * a + r] * inv;
    const int d0 = 32 * a + 16 * hf;
    if (p.out_bf16) {
      u32x4* dst = (u32x4*)(orow + 2 * d0);
      dst[0] = u32x4{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]), pack_bf16x2(v[4], v[5]), pack_bf16x2(v[6], v[7])};
      dst[1] = u32x4{pack_bf16x2(v[8], v[9]), pack_bf16x2(v[10], v[11]), pack_bf16x2(v[12], v[13]), pack_bf16x2(v[14], v[15])};
    } else {
      f32x4* dst = (f32x4*)(orow + 4 * d0);
      #pragma unroll
      for (int j = 0; j < 4; ++j) dst[j] = f32x4{v[4 * j], v[4 * j + 1], v[4 * j + 2], v[4 * j + 3]};
    }
  }
}

}  // namespace

hipError_t launch_prefill(const PrefillParams& p, hipStream_t stream) {
  const dim3 grid(p.n_qtiles * p.num_q_heads * p.batch);
  hipLaunchKernelGGL(prefill_kernel, grid, dim3(kThreads), 0, stream, p);
  return hipGetLastError();
}

}  // namespace gqa
