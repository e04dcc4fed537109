// Grouped-query causal prefill attention for gfx950 (MI355X) with the fused
// QK-norm + RoPE prologue on every query and key row.
//
// Algorithm (the pages):
//  * "ADR-0060: AHBM GQA Fused Attention Kernel (Llama3-70B)", section 3:
//    tiled online softmax (FlashAttention) over K/V tiles; section 5.4: a key
//    tile entirely in the future of a query block is skipped, one entirely in
//    its past needs no mask, an overlapping one gets the triangular mask, and
//    the query heads of one KV head are batched along the matrix M axis as in
//    decode (section 5.2: query head h reads KV head floor(h / G)).
//  * "Qwen3-14B Optimization", section 2.1 "Shape 4" / #796: QK-norm and RoPE
//    are applied inside the attention stage; #602: RoPE on lo/hi halves.
//
// gfx950 mapping:
//  * one workgroup = (sequence, KV head, a chunk of HC <= 8 of its query
//    heads, a block of BQ query tokens); wave w owns 32 query rows = one head
//    and 32 consecutive tokens, so a workgroup holds HC * BQ rows (10 waves for
//    5 heads x 64 tokens).  Every key tile, and its key prologue, is shared by
//    all of them.
//  * per 32-key tile: the raw K and V rows are fetched into registers one tile
//    ahead; K rows go through the key prologue (f32) and are stored as fp16 K'
//    in LDS (16-byte chunks XOR-swizzled by key), V rows are stored transposed
//    (V^T, key pairs packed per dword); both double-buffered, so one barrier
//    per tile suffices.  S^T = K' Q'^T and O^T = V^T P^T run on
//    v_mfma_f32_32x32x16_f16 with f32 accumulation; in the S^T orientation a
//    lane owns one query row, so the row max needs one cross-lane step.
//  * scores live in the log2 domain (scale * log2 e folded into the exp2 FMA);
//    the running output is rescaled only when a row maximum grows by more
//    than 2^8 (the final O / l is unchanged by the choice of reference max).
//  * a 1-D grid ordered so every (sequence, KV head) group lands on one XCD
//    (its K/V stay in that XCD's L2), heaviest query block first.
#include "common.hpp"

namespace gqa {
namespace {

constexpr int kMaxWaves = kPrefillMaxWaves;
constexpr int kMaxThreads = 64 * kMaxWaves;
constexpr int BN = 32;                 // keys per tile
constexpr int kXcds = 8;               // MI355X: 8 XCDs, each with its own L2
constexpr int kVtRow = 40;             // V^T row stride in fp16 (32 keys + 8): conflict-free 16-byte reads
constexpr float kLazyRescale = 8.0f;   // rescale O only when a row max grows by more than 2^8
constexpr int kKUnits = 256;           // K staging units per tile (32 keys x 8 dim chunks)
constexpr int kUnits = 512;            // + 256 V staging units (16 key pairs x 16 dim chunks)

struct __attribute__((aligned(16))) PrefillSmem {
  uint32_t kt[2][BN][kHeadDim / 2];   // K' tiles, fp16 pairs, 16-byte chunks swizzled by key & 15
  uint16_t vt[2][kHeadDim][kVtRow];   // V^T tiles: vt[buf][dim][vpos(key)]
  double inv_rev[kHeadDim / 2];       // theta^(-2i/128) / (2 pi)
  float gk[kHeadDim];                 // key RMSNorm weight (f32)
};

// Logical 16-byte chunk (of 16 per 128-dim row) holding operand slot kk of
// lane half hf: the lane's 8 slots cover dims [32hf, 32hf+32) and
// [64+32hf, 64+32hf+32), so every RoPE pair (i, i+64) stays in one lane.
__device__ __forceinline__ int qk_chunk(int kk, int hf) { return kk < 4 ? 4 * hf + kk : 8 + 4 * hf + (kk - 4); }

// Position of key k (0..31) of a tile in a V^T row.  Key 16e + 8a + 4h + r
// goes to 16e + 8h + 4a + r, so the 8 keys that MFMA e of lane half h takes
// ({16e + 4h + r, 16e + 8 + 4h + r}, r < 4) are 16 contiguous bytes.
__device__ __forceinline__ int vpos(int k) { return (k & 0x13) | ((k & 4) << 1) | ((k & 8) >> 1); }

// K' chunk swizzle: a bijection on keys mod 16 (conflict-free operand reads of
// 16 consecutive keys) that alternates the 128-byte half between neighbouring
// keys (fewer conflicts when 8 consecutive keys are stored together).
__device__ __forceinline__ int kswz(int key) { return (key & 15) ^ ((key & 1) << 3); }

struct Raw { u32x4 a, b; };

// One (sequence, KV head) slab: uniform 64-bit bases plus 32-bit byte offsets
// (the host guarantees each slab spans less than 4 GiB).
struct Staging {
  const uint8_t* kslab;
  const uint8_t* vslab;
  uint32_t kss, vss;   // row strides in bytes
  int n;
};

// Fetch staging unit u of tile kt.  K unit: key row u/8, dims [8(u%8), +8)
// and [64 + 8(u%8), +8).  V unit (u >= 256): key rows 2v, 2v+1 (v = (u-256)%16),
// dims [8((u-256)/16), +8).  Rows at or past n are zero (never read).
__device__ __forceinline__ void fetch_unit(Raw& r, const Staging& s, int kt, int u) {
  if (u < kKUnits) {
    const int key = kt * BN + (u >> 3), c = u & 7;
    if (key < s.n) {
      const uint32_t off = (uint32_t)key * s.kss + 16u * c;
      r.a = *(const u32x4*)(s.kslab + off);
      r.b = *(const u32x4*)(s.kslab + off + 128u);
    } else {
      r.a = r.b = u32x4{0, 0, 0, 0};
    }
  } else {
    const int v = u - kKUnits;
    const int key = kt * BN + 2 * (v & 15), dc = v >> 4;
    const uint32_t off = (uint32_t)key * s.vss + 16u * dc;
    r.a = key < s.n ? *(const u32x4*)(s.vslab + off) : u32x4{0, 0, 0, 0};
    r.b = key + 1 < s.n ? *(const u32x4*)(s.vslab + off + s.vss) : u32x4{0, 0, 0, 0};
  }
}

// Stage unit u of tile kt into LDS buffer buf: the key prologue for K units
// (RMSNorm over the row's 8 units = 8 consecutive lanes, then RoPE), the
// transpose for V units.
__device__ __forceinline__ void stage_unit(PrefillSmem& sm, const Raw& r, const PrefillParams& p, bool rope,
                                           double pos0, int kt, int u, int buf) {
  if (u < kKUnits) {
    const int lkey = u >> 3, c = u & 7;
    float xl[8], xh[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      xl[e] = bf16_elem(r.a, e);
      xh[e] = bf16_elem(r.b, e);
    }
    if (p.k_norm_w) {
      float ss = 0.f;
#pragma unroll
      for (int e = 0; e < 8; ++e) ss += xl[e] * xl[e] + xh[e] * xh[e];
      ss = sum8(ss);
      const float rr = 1.0f / sqrtf(ss * (1.0f / kHeadDim) + p.eps);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        xl[e] *= rr * sm.gk[8 * c + e];
        xh[e] *= rr * sm.gk[64 + 8 * c + e];
      }
    }
    if (rope) {
      const double kpos = pos0 + (double)(kt * BN + lkey);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        float cs, sn;
        rope_cos_sin_rev(kpos, sm.inv_rev[8 * c + e], cs, sn);
        const float lo = xl[e], hi = xh[e];
        xl[e] = lo * cs - hi * sn;
        xh[e] = hi * cs + lo * sn;
      }
    }
    uint32_t* krow = sm.kt[buf][lkey];
    const int sw = kswz(lkey);
    *(u32x4*)(krow + 4 * (c ^ sw)) = u32x4{pack_f16x2_sat(xl[0], xl[1]), pack_f16x2_sat(xl[2], xl[3]),
                                          pack_f16x2_sat(xl[4], xl[5]), pack_f16x2_sat(xl[6], xl[7])};
    *(u32x4*)(krow + 4 * ((8 + c) ^ sw)) = u32x4{pack_f16x2_sat(xh[0], xh[1]), pack_f16x2_sat(xh[2], xh[3]),
                                                pack_f16x2_sat(xh[4], xh[5]), pack_f16x2_sat(xh[6], xh[7])};
  } else {
    const int v = u - kKUnits;
    const int kp = v & 15, dc = v >> 4;
    const int pos = vpos(2 * kp);   // keys 2kp, 2kp+1 stay adjacent
#pragma unroll
    for (int j = 0; j < 4; ++j) {   // dims 8dc + 2j (lo halves) and 8dc + 2j + 1 (hi halves)
      const uint32_t a = r.a[j], c = r.b[j];
      *(uint32_t*)&sm.vt[buf][8 * dc + 2 * j][pos] = pack_f16x2_sat(bf16lo(a), bf16lo(c));
      *(uint32_t*)&sm.vt[buf][8 * dc + 2 * j + 1][pos] = pack_f16x2_sat(bf16hi(a), bf16hi(c));
    }
  }
}

// UNITS: staging units per thread per tile (1 when the workgroup has >= 8 waves, else 2).
template <int UNITS>
__global__ __launch_bounds__(kMaxThreads) void prefill_kernel(const PrefillParams p) {
  __shared__ PrefillSmem sm;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int nthreads = blockDim.x;
  const int n32 = lane & 31, hf = lane >> 5;
  const int G = p.group, HC = p.heads_per_wg, BQ = p.block_q;
  const int tb_per_head = BQ / 32;

  // ---- workgroup -> (sequence, KV head, head chunk, query block)
  const int nchunks = G / HC;
  const int per_group = p.n_qblocks * nchunks;
  const int groups = p.batch * p.num_kv_heads;
  const int bid = blockIdx.x;
  int grp, w;
  if (groups % kXcds == 0) {   // XCD-aware: a (sequence, KV head) group's workgroups share one XCD
    const int slot = bid / kXcds;
    grp = bid % kXcds + kXcds * (slot / per_group);
    w = slot % per_group;
  } else {
    grp = bid / per_group;
    w = bid % per_group;
  }
  const int b = grp / p.num_kv_heads, h = grp % p.num_kv_heads;
  const int qb = p.n_qblocks - 1 - w / nchunks;    // heaviest block first
  const int hc = w % nchunks;

  int n = p.seq_lens[b];
  n = n < 0 ? 0 : (n > p.max_seq ? p.max_seq : n);
  const int q0 = qb * BQ;
  if (q0 >= n) return;
  const int qe = min(q0 + BQ, n);
  const int kend = p.causal ? qe : n;              // keys [0, kend) can be visible
  const int ntiles = (kend + BN - 1) / BN;
  const bool rope = p.rope_theta > 0.0;
  const double pos0 = (double)p.positions[b];

  // this wave's rows: head hq, tokens [wq0, wq0 + 32)
  const int hq = h * G + hc * HC + wave / tb_per_head;
  const int wq0 = q0 + 32 * (wave % tb_per_head);
  const int qrow = wq0 + n32;
  const bool wave_live = wq0 < n;

  // ---- tables: RoPE inverse frequencies (revolutions) and key norm weight
  if (tid < 64 && rope) sm.inv_rev[tid] = rope_inv_freq(tid, p.rope_log2_theta) * 0.15915494309189535;
  if (tid < kHeadDim) sm.gk[tid] = p.k_norm_w ? bf16lo(((const uint16_t*)p.k_norm_w)[tid]) : 1.0f;

  Staging st;
  st.kslab = (const uint8_t*)p.k + ((int64_t)b * p.k_sb + (int64_t)h * p.k_sh) * 2;
  st.vslab = (const uint8_t*)p.v + ((int64_t)b * p.v_sb + (int64_t)h * p.v_sh) * 2;
  st.kss = (uint32_t)(p.k_ss * 2);
  st.vss = (uint32_t)(p.v_ss * 2);
  st.n = n;
  // staging units of this thread: tid and tid + nthreads (when below 512)
  const int u0 = tid, u1 = tid + nthreads;
  const bool has0 = u0 < kUnits, has1 = UNITS > 1 && u1 < kUnits;
  Raw r0, r1;

  // ---- fetch tile 0, run the query prologue, stage tile 0, fetch tile 1
  if (has0) fetch_unit(r0, st, 0, u0);
  if (has1) fetch_unit(r1, st, 0, u1);

  // query prologue: lane (n32, hf) owns row qrow of head hq, dims [32hf, 32hf+32) and [64+32hf, 64+32hf+32)
  f16x8 qf[8];
  {
    // raw row halves kept packed (16 registers each), unpacked chunk by chunk
    u32x4 qlo[4], qhi[4];
    if (qrow < n) {
      const uint16_t* row = (const uint16_t*)p.q + ((int64_t)b * p.q_sb + (int64_t)hq * p.q_sh + (int64_t)qrow * p.q_ss);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        qlo[j] = *(const u32x4*)(row + 32 * hf + 8 * j);
        qhi[j] = *(const u32x4*)(row + 64 + 32 * hf + 8 * j);
      }
    } else {
#pragma unroll
      for (int j = 0; j < 4; ++j) qlo[j] = qhi[j] = u32x4{0, 0, 0, 0};
    }
    float r = 1.0f;
    if (p.q_norm_w) {
      float ss = 0.f;
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float a = bf16_elem(qlo[j], e), c = bf16_elem(qhi[j], e);
          ss += a * a + c * c;
        }
      ss = sum_xor32(ss);
      r = 1.0f / sqrtf(ss * (1.0f / kHeadDim) + p.eps);
    }
    __syncthreads();   // the tables are written
    const double qpos = pos0 + (double)qrow;
    const uint16_t* g = (const uint16_t*)p.q_norm_w;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      float xl[8], xh[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        xl[e] = bf16_elem(qlo[j], e);
        xh[e] = bf16_elem(qhi[j], e);
      }
      if (g) {
        const u32x4 glo = *(const u32x4*)(g + 32 * hf + 8 * j);
        const u32x4 ghi = *(const u32x4*)(g + 64 + 32 * hf + 8 * j);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          xl[e] *= r * bf16_elem(glo, e);
          xh[e] *= r * bf16_elem(ghi, e);
        }
      }
      if (rope) {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          float c, s;
          rope_cos_sin_rev(qpos, sm.inv_rev[32 * hf + 8 * j + e], c, s);
          const float lo = xl[e], hi = xh[e];
          xl[e] = lo * c - hi * s;
          xh[e] = hi * c + lo * s;
        }
      }
      qf[j] = as_f16x8(u32x4{pack_f16x2_sat(xl[0], xl[1]), pack_f16x2_sat(xl[2], xl[3]),
                              pack_f16x2_sat(xl[4], xl[5]), pack_f16x2_sat(xl[6], xl[7])});
      qf[4 + j] = as_f16x8(u32x4{pack_f16x2_sat(xh[0], xh[1]), pack_f16x2_sat(xh[2], xh[3]),
                                  pack_f16x2_sat(xh[4], xh[5]), pack_f16x2_sat(xh[6], xh[7])});
    }
  }
  if (has0) stage_unit(sm, r0, p, rope, pos0, 0, u0, 0);
  if (has1) stage_unit(sm, r1, p, rope, pos0, 0, u1, 0);
  if (ntiles > 1) {
    if (has0) fetch_unit(r0, st, 1, u0);
    if (has1) fetch_unit(r1, st, 1, u1);
  }
  __syncthreads();   // tile 0 staged

  f32x16 o[4];
#pragma unroll
  for (int T = 0; T < 4; ++T)
#pragma unroll
    for (int i = 0; i < 16; ++i) o[T][i] = 0.f;
  float m_run = -INFINITY, l_run = 0.f;

  for (int kt = 0; kt < ntiles; ++kt) {
    const int buf = kt & 1;
    // ---- attention on tile kt for this wave's 32 query rows
    const int ks = kt * BN;
    const bool future = p.causal && ks > wq0 + 31;
    if (wave_live && !future) {
      // sacc[i] = S[key ks + 8(i/4) + 4hf + i%4][query wq0 + n32] (raw, unscaled)
      f32x16 sacc;
#pragma unroll
      for (int i = 0; i < 16; ++i) sacc[i] = 0.f;
      {
        const uint32_t* kr = sm.kt[buf][n32];
        const int sw = kswz(n32);
#pragma unroll
        for (int kk = 0; kk < 8; ++kk) {
          const u32x4 a = *(const u32x4*)(kr + 4 * (qk_chunk(kk, hf) ^ sw));
          sacc = __builtin_amdgcn_mfma_f32_32x32x16_f16(as_f16x8(a), qf[kk], sacc, 0, 0, 0);
        }
      }
      if ((p.causal && ks + BN - 1 > wq0) || ks + BN > n) {   // wave-uniform: diagonal or ragged tile
        // key ks + off is visible iff off < lim (off = 8(i/4) + 4hf + i%4)
        const int lim = (p.causal ? min(n, qrow + 1) : n) - ks - 4 * hf;
#pragma unroll
        for (int i = 0; i < 16; ++i) sacc[i] = (8 * (i >> 2) + (i & 3) < lim) ? sacc[i] : -INFINITY;
      }
      // IEEE maximum trees (no quieting of the MFMA results), then one maximum
      // across the two lane halves that hold the row's two key halves
      float mx = sacc[0];
#pragma unroll
      for (int i = 1; i < 15; i += 2)
        mx = __builtin_elementwise_maximum(__builtin_elementwise_maximum(mx, sacc[i]), sacc[i + 1]);
      mx = __builtin_elementwise_maximum(mx, sacc[15]);
      {
        float a, b;
        pair_xor32(mx, a, b);
        mx = __builtin_elementwise_maximum(a, b) * p.scale_log2;   // row max in log2 units
      }
      // lazy rescale: keep the running max until some row's max grows by more
      // than kLazyRescale; exponents stay <= 2^kLazyRescale meanwhile
      if (__any(mx > m_run + kLazyRescale)) {
        const float m_new = fmaxf(m_run, mx);
        const float corr = fast_exp2(m_run - m_new);   // 0 on the first tile (m = -inf)
        l_run *= corr;
#pragma unroll
        for (int T = 0; T < 4; ++T) o[T] *= corr;
        m_run = m_new;
      }
#pragma unroll
      for (int i = 0; i < 16; ++i) sacc[i] = fast_exp2(fmaf(sacc[i], p.scale_log2, -m_run));
      // O^T += V^T P^T: MFMA e takes keys ks + 16e + {4hf + t, 8 + 4hf + t}, t < 4,
      // stored contiguously at V^T positions 16e + 8hf .. 16e + 8hf + 7.  The
      // row sum is taken over the fp16 P the products use (v_dot2 of each
      // pair with (1, 1)), so numerator and denominator see the same weights.
      const f16x2 one = {(_Float16)1.0f, (_Float16)1.0f};
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        const u32x4 pf = {pack_f16x2(sacc[8 * e + 0], sacc[8 * e + 1]), pack_f16x2(sacc[8 * e + 2], sacc[8 * e + 3]),
                          pack_f16x2(sacc[8 * e + 4], sacc[8 * e + 5]), pack_f16x2(sacc[8 * e + 6], sacc[8 * e + 7])};
#pragma unroll
        for (int w = 0; w < 4; ++w)   // the (uint32_t) copy matters: hipcc bit-casts element 0 of a vector lvalue
          l_run = __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2, (uint32_t)pf[w]), one, l_run, false);
#pragma unroll
        for (int T = 0; T < 4; ++T) {
          const u32x4 a = *(const u32x4*)&sm.vt[buf][32 * T + n32][16 * e + 8 * hf];
          o[T] = __builtin_amdgcn_mfma_f32_32x32x16_f16(as_f16x8(a), as_f16x8(pf), o[T], 0, 0, 0);
        }
      }
    }
    // ---- stage tile kt+1 into the other buffer (nobody reads it since the last
    //      barrier); placed after the P V MFMAs are issued so that this VALU
    //      work overlaps them
    if (kt + 1 < ntiles) {
      if (has0) stage_unit(sm, r0, p, rope, pos0, kt + 1, u0, buf ^ 1);
      if (has1) stage_unit(sm, r1, p, rope, pos0, kt + 1, u1, buf ^ 1);
      if (kt + 2 < ntiles) {
        if (has0) fetch_unit(r0, st, kt + 2, u0);
        if (has1) fetch_unit(r1, st, kt + 2, u1);
      }
    }
    __syncthreads();
  }

  // ---- epilogue: O / l for this lane's query row
  if (!wave_live || qrow >= n) return;
  l_run = sum_xor32(l_run);
  const float inv = 1.0f / l_run;
  uint8_t* orow = (uint8_t*)p.out + ((int64_t)b * p.o_sb + (int64_t)hq * p.o_sh + (int64_t)qrow * p.o_ss) * (p.out_bf16 ? 2 : 4);
  // o[T][4a + r] = O[query][dim 32T + 8a + 4hf + r]
#pragma unroll
  for (int T = 0; T < 4; ++T) {
#pragma unroll
    for (int a = 0; a < 4; ++a) {
      const int d0 = 32 * T + 8 * a + 4 * hf;
      const float v0 = o[T][4 * a] * inv, v1 = o[T][4 * a + 1] * inv, v2 = o[T][4 * a + 2] * inv, v3 = o[T][4 * a + 3] * inv;
      if (p.out_bf16) *(u32x2*)(orow + 2 * d0) = u32x2{pack_bf16x2(v0, v1), pack_bf16x2(v2, v3)};
      else *(f32x4*)(orow + 4 * d0) = f32x4{v0, v1, v2, v3};
    }
  }
}

}  // namespace

hipError_t launch_prefill_fused(const PrefillParams& p, hipStream_t stream) {
  const int waves = p.heads_per_wg * p.block_q / 32;
  const dim3 grid(p.n_qblocks * (p.group / p.heads_per_wg) * p.num_kv_heads * p.batch);
  if (64 * waves >= kUnits) return launch_kernel(prefill_kernel<1>, grid, dim3(64 * waves), stream, p);
  return launch_kernel(prefill_kernel<2>, grid, dim3(64 * waves), stream, p);
}

}  // namespace gqa
