// Grouped-query decode attention for gfx950 (MI355X): split-KV partition
// kernel with the fused QK-norm + RoPE prologue, and the log-sum-exp merge.
//
// Algorithm (the pages):
//  * "ADR-0060: AHBM GQA Fused Attention Kernel (Llama3-70B)", section 5.2:
//    the G query heads of one KV head are folded into the matrix M dimension
//    so that one K/V tile read from memory serves all G heads; section 3:
//    per K/V tile, S = scale * Q K^T, running max m, P = exp(S - m_new),
//    corr = exp(m - m_new), l = l*corr + sum P, O = O*corr + P V, seeded
//    (-inf, 0, 0); section 4: split partials (m, l, O) are combined by the
//    log-sum-exp merge and normalised once; section 2.2: chunk c of a
//    sequence covers a contiguous block of keys.
//  * "Qwen3-14B Optimization", section 2.1 "Shape 4" / #796: QK-norm and
//    RoPE run inside the attention stage; #602: RoPE on lo/hi halves.
//
// gfx950 mapping (not the pages' design, which targets an NPU / simulator):
//  * one workgroup = (chunk c, KV head h, sequence b), 4 waves of 64 lanes;
//    wave w handles 32-key steps w, w+4, ... of the chunk and keeps its own
//    online-softmax state; the 4 states are merged through LDS at the end.
//  * S^T = K Q'^T and O^T = V^T P^T run on v_mfma_f32_16x16x32_bf16 (bf16
//    inputs) or v_mfma_f32_16x16x4_f32 (f32 inputs) with the G <= 16 query
//    rows as the 16-wide N dimension.  In this orientation a lane owns one
//    query head (lane % 16), so the row max needs only two cross-lane steps,
//    and V rows are read with 16 lanes covering one full 256-byte row; the
//    8x8 bf16 transpose that V^T needs is done in registers.
//  * K and V are streamed straight from HBM into registers: the first step is
//    requested before the query prologue runs, and each step buffer is
//    refilled with the wave's next step as soon as its K (then V) half has
//    been consumed.
#include "common.hpp"

namespace gqa {
namespace {

constexpr int kWaves = 4;
constexpr int kThreads = kWaves * 64;
constexpr int kStep = 32;        // keys per wave step
constexpr int kORow = 132;       // padded LDS row (floats) of the in-workgroup merge

struct DecodeSmem {
  float cs[64][2];               // RoPE cos / sin at positions[b]
  float qp[16][kHeadDim];        // q' rows after the prologue (rows >= G are zero)
  float kn[kHeadDim];            // the new key row after the prologue
  float mo[kWaves][16][kORow];   // per-wave unnormalised O (in-workgroup merge)
  float mm[kWaves][16];
  float ml[kWaves][16];
};

template <bool BF16>
__device__ __forceinline__ void load_half_row(const void* row, int c16, float (&x)[8]) {
  // x[0..3] = dims 4*c16 .. 4*c16+3; x[4..7] = dims 64+4*c16 .. 64+4*c16+3
  if constexpr (BF16) {
    const uint16_t* r = (const uint16_t*)row;
    const u32x2 lo = *(const u32x2*)(r + 4 * c16);
    const u32x2 hi = *(const u32x2*)(r + 64 + 4 * c16);
    x[0] = bf16lo(lo[0]); x[1] = bf16hi(lo[0]); x[2] = bf16lo(lo[1]); x[3] = bf16hi(lo[1]);
    x[4] = bf16lo(hi[0]); x[5] = bf16hi(hi[0]); x[6] = bf16lo(hi[1]); x[7] = bf16hi(hi[1]);
  } else {
    const float* r = (const float*)row;
    const f32x4 lo = *(const f32x4*)(r + 4 * c16);
    const f32x4 hi = *(const f32x4*)(r + 64 + 4 * c16);
    #pragma unroll
    for (int j = 0; j < 4; ++j) { x[j] = lo[j]; x[4 + j] = hi[j]; }
  }
}

// The prologue on one row held by 16 consecutive lanes (8 elements each):
// RMSNorm over the 128 elements (skipped if gamma is null), then RoPE with
// the cos/sin table (skipped if !rope).  All 16 lanes must be active.
template <bool BF16>
__device__ __forceinline__ void prologue_row(float (&x)[8], int c16, const void* gamma, float eps, bool rope,
                                             const float (*cs)[2]) {
  if (gamma != nullptr) {
    float ss = 0.f;
    #pragma unroll
    for (int j = 0; j < 8; ++j) ss += x[j] * x[j];
    ss += __shfl_xor(ss, 1, 16);
    ss += __shfl_xor(ss, 2, 16);
    ss += __shfl_xor(ss, 4, 16);
    ss += __shfl_xor(ss, 8, 16);
    const float r = 1.0f / sqrtf(ss * (1.0f / kHeadDim) + eps);
    float g[8];
    load_half_row<BF16>(gamma, c16, g);
    #pragma unroll
    for (int j = 0; j < 8; ++j) x[j] = x[j] * r * g[j];
  }
  if (rope) {
    #pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float c = cs[4 * c16 + j][0], s = cs[4 * c16 + j][1];
      const float lo = x[j], hi = x[4 + j];
      x[j] = lo * c - hi * s;
      x[4 + j] = hi * c + lo * s;
    }
  }
}

// ----------------------------------------------------------------- K/V step buffers

struct StepBF16 {
  u32x4 k[2][4];   // K rows key0 + 16*gi + (lane%16), dims 32*(lane/16) + 8*kb .. +8
  u32x4 v[8];      // V rows key0 + vkey(t), dims 8*(lane%16) .. +8
};

struct StepF32 {
  f32x4 k[2][8];   // K rows key0 + 16*gi + (lane%16), dims 32*(lane/16) .. +32
  f32x4 v[8][2];   // V rows key0 + 16*gi + 4*(lane/16) + i (e = 4*gi + i), dims 8*(lane%16) .. +8
};

// key offset (within a 32-key step) of the t-th V row a bf16 lane loads; the
// same permutation orders the P^T operand: t < 4 -> 4*q4 + t, else 16 + 4*q4 + t - 4
__device__ __forceinline__ constexpr int vkey_t(int t) { return t < 4 ? t : 12 + t; }

// Addressing of one (b, KV head) slab: a uniform 64-bit base plus 32-bit byte
// offsets (the host guarantees the slab spans less than 4 GiB).  The per-lane
// parts of the offsets are fixed for the whole sweep.
struct Slab {
  const uint8_t* kb;
  const uint8_t* vb;
  uint32_t kss, vss;     // row strides in bytes
  uint32_t klane, vlane; // per-lane byte offsets
};

// Loads of one step.  FULL: every row of the step is below kend, no
// predication.  !FULL (the last step of a chunk): rows at or past kend are
// replaced by row kend-1 (always valid) and the loaded values are zeroed, so
// rows past the sequence are never read and the code stays branch-free.
template <bool FULL>
__device__ __forceinline__ void load_k(StepBF16& st, const Slab& sl, int key0, int kend, int n16, int q4) {
#pragma unroll
  for (int gi = 0; gi < 2; ++gi) {
    const int key = key0 + 16 * gi + n16;
    const bool ok = FULL || key < kend;
    const uint32_t off = FULL ? (uint32_t)(key0 + 16 * gi) * sl.kss + sl.klane
                              : (uint32_t)(ok ? key : kend - 1) * sl.kss + 64u * q4;
    const u32x4* src = (const u32x4*)(sl.kb + off);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const u32x4 x = src[j];
      st.k[gi][j] = ok ? x : u32x4{0, 0, 0, 0};
    }
  }
}

template <bool FULL>
__device__ __forceinline__ void load_v(StepBF16& st, const Slab& sl, int key0, int kend, int n16, int q4) {
#pragma unroll
  for (int t = 0; t < 8; ++t) {
    const int key = key0 + 4 * q4 + vkey_t(t);
    const bool ok = FULL || key < kend;
    const uint32_t off = FULL ? (uint32_t)(key0 + vkey_t(t)) * sl.vss + sl.vlane
                              : (uint32_t)(ok ? key : kend - 1) * sl.vss + 16u * n16;
    const u32x4 x = *(const u32x4*)(sl.vb + off);
    st.v[t] = ok ? x : u32x4{0, 0, 0, 0};
  }
}

template <bool FULL>
__device__ __forceinline__ void load_k(StepF32& st, const Slab& sl, int key0, int kend, int n16, int q4) {
#pragma unroll
  for (int gi = 0; gi < 2; ++gi) {
    const int key = key0 + 16 * gi + n16;
    const bool ok = FULL || key < kend;
    const uint32_t off = FULL ? (uint32_t)(key0 + 16 * gi) * sl.kss + sl.klane
                              : (uint32_t)(ok ? key : kend - 1) * sl.kss + 128u * q4;
    const f32x4* src = (const f32x4*)(sl.kb + off);
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const f32x4 x = src[j];
      st.k[gi][j] = ok ? x : f32x4{0.f, 0.f, 0.f, 0.f};
    }
  }
}

template <bool FULL>
__device__ __forceinline__ void load_v(StepF32& st, const Slab& sl, int key0, int kend, int n16, int q4) {
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const int key = key0 + 16 * (e >> 2) + 4 * q4 + (e & 3);
    const bool ok = FULL || key < kend;
    const uint32_t off = FULL ? (uint32_t)(key0 + 16 * (e >> 2) + (e & 3)) * sl.vss + sl.vlane
                              : (uint32_t)(ok ? key : kend - 1) * sl.vss + 32u * n16;
    const f32x4* src = (const f32x4*)(sl.vb + off);
    const f32x4 x0 = src[0], x1 = src[1];
    st.v[e][0] = ok ? x0 : f32x4{0.f, 0.f, 0.f, 0.f};
    st.v[e][1] = ok ? x1 : f32x4{0.f, 0.f, 0.f, 0.f};
  }
}

template <class Step>
__device__ __forceinline__ void load_k_any(Step& st, const Slab& sl, int key0, int kend, int n16, int q4) {
  if (key0 + kStep <= kend) load_k<true>(st, sl, key0, kend, n16, q4);
  else load_k<false>(st, sl, key0, kend, n16, q4);
}

template <class Step>
__device__ __forceinline__ void load_v_any(Step& st, const Slab& sl, int key0, int kend, int n16, int q4) {
  if (key0 + kStep <= kend) load_v<true>(st, sl, key0, kend, n16, q4);
  else load_v<false>(st, sl, key0, kend, n16, q4);
}

template <class Step>
__device__ __forceinline__ void load_step(Step& st, const Slab& sl, int key0, int kend, int n16, int q4) {
  load_k_any(st, sl, key0, kend, n16, q4);
  load_v_any(st, sl, key0, kend, n16, q4);
}

// ----------------------------------------------------------------- query operand and running state

// bf16 path: q' = hi + lo with hi = bf16(q'), lo = bf16(q' - hi), so the score
// keeps ~16 significant bits of q' (two MFMAs per product; decode has the
// matrix-core headroom).
struct QFragBF16 { bf16x8 hi[4], lo[4]; };
struct QFragF32 { float q[32]; };

struct RunState {
  f32x4 o[8];      // O^T tiles: lane holds O[g = lane%16][dim (4*(lane/16)+i)*8 + T] in o[T][i]
  float m;         // running max (log2 units), same in the 4 lanes of one query head
  float l;         // this lane's share of the running normaliser
};

// scores: s[4*gi + i] = S[key key0 + 16*gi + 4*q4 + i][g = lane%16] (log2 units).
// nk_gi >= 0 (wave-uniform): the step holds the new key (slot L-1) in group
// nk_gi; the lane whose row it is (nk_lane) uses its prologue output, read
// from LDS, instead of the raw cached row.
__device__ __forceinline__ void scores(const StepBF16& st, const QFragBF16& qf, const float* knl, int nk_gi,
                                       bool nk_lane, int q4, float scale_log2, float (&s)[8]) {
#pragma unroll
  for (int gi = 0; gi < 2; ++gi) {
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    if (nk_gi == gi) {
      // K'_new = hi + lo: hi replaces the raw row, lo adds one more product
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) {
        const float* x = knl + 32 * q4 + 8 * kb;
        float hv[8], lv[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          hv[j] = (float)(__bf16)x[j];
          lv[j] = nk_lane ? x[j] - hv[j] : 0.f;
        }
        const u32x4 hi = {pack_bf16x2(hv[0], hv[1]), pack_bf16x2(hv[2], hv[3]), pack_bf16x2(hv[4], hv[5]),
                          pack_bf16x2(hv[6], hv[7])};
        const u32x4 lo = {pack_bf16x2(lv[0], lv[1]), pack_bf16x2(lv[2], lv[3]), pack_bf16x2(lv[4], lv[5]),
                          pack_bf16x2(lv[6], lv[7])};
        const u32x4 a = nk_lane ? hi : st.k[gi][kb];
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(a), qf.hi[kb], acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(a), qf.lo[kb], acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(lo), qf.hi[kb], acc, 0, 0, 0);
      }
    } else {
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) {
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(st.k[gi][kb]), qf.hi[kb], acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(st.k[gi][kb]), qf.lo[kb], acc, 0, 0, 0);
      }
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) s[4 * gi + i] = acc[i] * scale_log2;
  }
}

__device__ __forceinline__ void scores(const StepF32& st, const QFragF32& qf, const float* knl, int nk_gi,
                                       bool nk_lane, int q4, float scale_log2, float (&s)[8]) {
#pragma unroll
  for (int gi = 0; gi < 2; ++gi) {
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    const bool sub = nk_gi == gi && nk_lane;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      f32x4 a = st.k[gi][j];
      if (sub) {
        const float* x = knl + 32 * q4 + 4 * j;
        a = f32x4{x[0], x[1], x[2], x[3]};
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a[e], qf.q[4 * j + e], acc, 0, 0, 0);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) s[4 * gi + i] = acc[i] * scale_log2;
  }
}

// O^T += V^T P^T.  bf16 path: P = hi + lo (two MFMAs per tile).
__device__ __forceinline__ void accumulate_pv(const StepBF16& st, const float (&p)[8], RunState& rs) {
  // P^T operand: slot t of lane group q4 <-> key vkey_bf16(q4, t) = the score
  // order p[0..7] of this lane.
  float h[8], r[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    h[e] = (float)(__bf16)p[e];
    r[e] = p[e] - h[e];
  }
  const u32x4 phi = {pack_bf16x2(h[0], h[1]), pack_bf16x2(h[2], h[3]), pack_bf16x2(h[4], h[5]), pack_bf16x2(h[6], h[7])};
  const u32x4 plo = {pack_bf16x2(r[0], r[1]), pack_bf16x2(r[2], r[3]), pack_bf16x2(r[4], r[5]), pack_bf16x2(r[6], r[7])};
#pragma unroll
  for (int T = 0; T < 8; ++T) {
    const int w = T >> 1;
    u32x4 a;
#pragma unroll
    for (int u = 0; u < 4; ++u)
      a[u] = (T & 1) ? pair_hi(st.v[2 * u][w], st.v[2 * u + 1][w]) : pair_lo(st.v[2 * u][w], st.v[2 * u + 1][w]);
    rs.o[T] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(a), as_bf16x8(phi), rs.o[T], 0, 0, 0);
    rs.o[T] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(a), as_bf16x8(plo), rs.o[T], 0, 0, 0);
  }
}

__device__ __forceinline__ void accumulate_pv(const StepF32& st, const float (&p)[8], RunState& rs) {
#pragma unroll
  for (int e = 0; e < 8; ++e)
#pragma unroll
    for (int T = 0; T < 8; ++T)
      rs.o[T] = __builtin_amdgcn_mfma_f32_16x16x4f32(st.v[e][T >> 2][T & 3], p[e], rs.o[T], 0, 0, 0);
}

// One 32-key step from buffer st; afterwards st is refilled with the step at
// next_key0 (if next_key0 < kend): its K half right after the QK^T MFMAs
// have consumed st.k, its V half right after P V has consumed st.v.
template <class Step, class QFrag>
__device__ __forceinline__ void sweep_step(Step& st, const QFrag& qf, const float* knl, bool has_new, int kn,
                                           RunState& rs, float scale_log2, int key0, int kend, int next_key0,
                                           const Slab& sl, int n16, int q4) {
  const bool full = key0 + kStep <= kend;
  int nk_gi = -1;
  bool nk_lane = false;
  if (has_new && kn >= key0 && kn < key0 + kStep) {   // wave-uniform
    nk_gi = (kn - key0) >> 4;
    nk_lane = ((kn - key0) & 15) == n16;
  }
  float s[8];
  scores(st, qf, knl, nk_gi, nk_lane, q4, scale_log2, s);
  const bool more = next_key0 < kend;
  if (more) load_k_any(st, sl, next_key0, kend, n16, q4);
  if (!full) {
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int key = key0 + 16 * (e >> 2) + 4 * q4 + (e & 3);
      if (key >= kend) s[e] = -INFINITY;
    }
  }
  float mx = s[0];
#pragma unroll
  for (int e = 1; e < 8; ++e) mx = fmaxf(mx, s[e]);
  mx = wave_max_xor(mx, 16);
  mx = wave_max_xor(mx, 32);
  const float m_new = fmaxf(rs.m, mx);
  const float corr = fast_exp2(rs.m - m_new);   // 0 on the first step (m = -inf)
  float p[8];
  float ps = 0.f;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    p[e] = fast_exp2(s[e] - m_new);
    ps += p[e];
  }
  rs.l = rs.l * corr + ps;
  rs.m = m_new;
#pragma unroll
  for (int T = 0; T < 8; ++T) rs.o[T] *= corr;
  accumulate_pv(st, p, rs);
  if (more) load_v_any(st, sl, next_key0, kend, n16, q4);
}

template <bool BF16>
__global__ __launch_bounds__(kThreads, 2) void decode_partition_kernel(const DecodeParams p) {
  using Step = typename std::conditional<BF16, StepBF16, StepF32>::type;
  using QFrag = typename std::conditional<BF16, QFragBF16, QFragF32>::type;
  constexpr int kElem = BF16 ? 2 : 4;

  __shared__ DecodeSmem sm;

  const int c = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int n16 = lane & 15, q4 = lane >> 4;
  const int G = p.group;
  const bool direct = p.n_split == 1;

  int L = p.seq_lens[b];
  L = L < 0 ? 0 : (L > p.max_seq ? p.max_seq : L);
  const int c0 = c * p.split;
  if (c0 >= L) {
    if (direct && c == 0) {   // L == 0: defined as an all-zero output row
      const int g = tid >> 4, d8 = (tid & 15) * 8;
      if (g < G) {
        uint8_t* o = (uint8_t*)p.out + ((int64_t)b * p.o_sb + (int64_t)(h * G + g) * p.o_sh) * (p.out_bf16 ? 2 : 4);
        if (p.out_bf16) {
          *(u32x4*)(o + 2 * d8) = u32x4{0, 0, 0, 0};
        } else {
          *(f32x4*)(o + 4 * d8) = f32x4{0.f, 0.f, 0.f, 0.f};
          *(f32x4*)(o + 4 * d8 + 16) = f32x4{0.f, 0.f, 0.f, 0.f};
        }
      }
    }
    return;
  }
  const int c1 = min(c0 + p.split, L);
  const int nsteps = (c1 - c0 + kStep - 1) / kStep;
  Slab sl;
  sl.kb = (const uint8_t*)p.k + ((int64_t)b * p.k_sb + (int64_t)h * p.k_sh) * kElem;
  sl.vb = (const uint8_t*)p.v + ((int64_t)b * p.v_sb + (int64_t)h * p.v_sh) * kElem;
  sl.kss = (uint32_t)(p.k_ss * kElem);
  sl.vss = (uint32_t)(p.v_ss * kElem);
  if constexpr (BF16) {
    sl.klane = (uint32_t)n16 * sl.kss + 64u * q4;          // K row n16, dims 32*q4 ..
    sl.vlane = (uint32_t)(4 * q4) * sl.vss + 16u * n16;    // V rows 4*q4 + .., dims 8*n16 ..
  } else {
    sl.klane = (uint32_t)n16 * sl.kss + 128u * q4;
    sl.vlane = (uint32_t)(4 * q4) * sl.vss + 32u * n16;
  }

  // ---- the first K/V steps go to memory before anything else, so that their
  //      latency overlaps the query prologue
  int s = wave;
  Step A;
  if (s < nsteps) load_step(A, sl, c0 + s * kStep, c1, n16, q4);

  const bool rope = p.rope_theta > 0.0;
  const bool k_pro = rope || p.k_norm_w != nullptr;
  const bool has_new = k_pro && c1 == L;   // this chunk holds slot L-1
  const double pos = (double)p.positions[b];

  // ---- prologue: RoPE table, q' (and the new key row) into LDS
  if (rope && tid < 64) rope_cos_sin_f64(pos, tid, p.rope_theta, sm.cs[tid][0], sm.cs[tid][1]);
  __syncthreads();
  {
    const int r = tid >> 4, c16 = tid & 15;
    float x[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    if (r < G) {
      const uint8_t* row = (const uint8_t*)p.q + ((int64_t)b * p.q_sb + (int64_t)(h * G + r) * p.q_sh) * kElem;
      load_half_row<BF16>(row, c16, x);
    }
    prologue_row<BF16>(x, c16, p.q_norm_w, p.eps, rope, sm.cs);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      sm.qp[r][4 * c16 + j] = x[j];
      sm.qp[r][64 + 4 * c16 + j] = x[4 + j];
    }
    if (has_new && tid < 16) {
      const uint8_t* row = (const uint8_t*)p.k + ((int64_t)b * p.k_sb + (int64_t)h * p.k_sh + (int64_t)(L - 1) * p.k_ss) * kElem;
      float y[8];
      load_half_row<BF16>(row, c16, y);
      prologue_row<BF16>(y, c16, p.k_norm_w, p.eps, rope, sm.cs);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        sm.kn[4 * c16 + j] = y[j];
        sm.kn[64 + 4 * c16 + j] = y[4 + j];
      }
    }
  }
  __syncthreads();

  QFrag qf;
  if constexpr (BF16) {
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
      const float* x = &sm.qp[n16][32 * q4 + 8 * kb];
      float hi[8], lo[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        hi[j] = (float)(__bf16)x[j];
        lo[j] = x[j] - hi[j];
      }
      qf.hi[kb] = as_bf16x8(u32x4{pack_bf16x2(hi[0], hi[1]), pack_bf16x2(hi[2], hi[3]), pack_bf16x2(hi[4], hi[5]),
                                  pack_bf16x2(hi[6], hi[7])});
      qf.lo[kb] = as_bf16x8(u32x4{pack_bf16x2(lo[0], lo[1]), pack_bf16x2(lo[2], lo[3]), pack_bf16x2(lo[4], lo[5]),
                                  pack_bf16x2(lo[6], lo[7])});
    }
  } else {
#pragma unroll
    for (int j = 0; j < 32; ++j) qf.q[j] = sm.qp[n16][32 * q4 + j];
  }
  const int kn = L - 1;

  // ---- the sweep over this chunk's keys
  RunState rs;
#pragma unroll
  for (int T = 0; T < 8; ++T) rs.o[T] = f32x4{0.f, 0.f, 0.f, 0.f};
  rs.m = -INFINITY;
  rs.l = 0.f;

  // one step buffer per wave, refilled in place: the next step's K is in
  // flight during this step's softmax and P V, its V during the next QK^T
  while (s < nsteps) {
    sweep_step(A, qf, sm.kn, has_new, kn, rs, p.scale_log2, c0 + s * kStep, c1, c0 + (s + kWaves) * kStep, sl, n16,
               q4);
    s += kWaves;
  }

  // ---- merge the 4 wave states of this workgroup (ADR-0060 section 4 merge)
  rs.l = wave_sum_xor(rs.l, 16);
  rs.l = wave_sum_xor(rs.l, 32);
  if (q4 == 0) {
    sm.mm[wave][n16] = rs.m;
    sm.ml[wave][n16] = rs.l;
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    float* dst = &sm.mo[wave][n16][(4 * q4 + i) * 8];
    *(f32x4*)dst = f32x4{rs.o[0][i], rs.o[1][i], rs.o[2][i], rs.o[3][i]};
    *(f32x4*)(dst + 4) = f32x4{rs.o[4][i], rs.o[5][i], rs.o[6][i], rs.o[7][i]};
  }
  __syncthreads();

  const int g = tid >> 4, d8 = (tid & 15) * 8;
  if (g >= G) return;
  float M = sm.mm[0][g];
#pragma unroll
  for (int w = 1; w < kWaves; ++w) M = fmaxf(M, sm.mm[w][g]);
  float lt = 0.f;
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int w = 0; w < kWaves; ++w) {
    const float sc = fast_exp2(sm.mm[w][g] - M);   // 0 for a wave that saw no key
    lt += sc * sm.ml[w][g];
    const float* src = &sm.mo[w][g][d8];
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[j] += sc * src[j];
  }
  const int hq = h * G + g;
  if (direct) {
    const float inv = 1.0f / lt;
    uint8_t* o = (uint8_t*)p.out + ((int64_t)b * p.o_sb + (int64_t)hq * p.o_sh) * (p.out_bf16 ? 2 : 4);
    if (p.out_bf16) {
      *(u32x4*)(o + 2 * d8) = u32x4{pack_bf16x2(acc[0] * inv, acc[1] * inv), pack_bf16x2(acc[2] * inv, acc[3] * inv),
                                    pack_bf16x2(acc[4] * inv, acc[5] * inv), pack_bf16x2(acc[6] * inv, acc[7] * inv)};
    } else {
      *(f32x4*)(o + 4 * d8) = f32x4{acc[0] * inv, acc[1] * inv, acc[2] * inv, acc[3] * inv};
      *(f32x4*)(o + 4 * d8 + 16) = f32x4{acc[4] * inv, acc[5] * inv, acc[6] * inv, acc[7] * inv};
    }
  } else {
    const int64_t slot = ((int64_t)b * p.num_q_heads + hq) * p.n_split + c;
    float* wo = p.ws_o + slot * kHeadDim + d8;
    *(f32x4*)wo = f32x4{acc[0], acc[1], acc[2], acc[3]};
    *(f32x4*)(wo + 4) = f32x4{acc[4], acc[5], acc[6], acc[7]};
    if ((tid & 15) == 0) {
      p.ws_ml[2 * slot] = M;
      p.ws_ml[2 * slot + 1] = lt;
    }
  }
}

// ----------------------------------------------------------------- merge kernel
// One workgroup per (q head, sequence): out = sum_c 2^(m_c - M) O_c / sum_c 2^(m_c - M) l_c
// over the n = ceil(L / T) chunks that hold keys (ADR-0060 section 4).  Thread
// (group sg, dims 4*d4 .. 4*d4+3) folds chunks sg, sg + 16, ... with a running
// maximum, kMergeUnroll chunks per batch of loads; the 16 group states are then
// merged through LDS.

constexpr int kMergeThreads = 512;
constexpr int kMergeGroups = kMergeThreads / 32;
constexpr int kMergeUnroll = 8;

__global__ __launch_bounds__(kMergeThreads) void decode_merge_kernel(const DecodeParams p) {
  __shared__ __attribute__((aligned(16))) float racc[kMergeGroups][kHeadDim];
  __shared__ float rm[kMergeGroups], rl[kMergeGroups];

  const int hq = blockIdx.x, b = blockIdx.y, tid = threadIdx.x;
  int L = p.seq_lens[b];
  L = L < 0 ? 0 : (L > p.max_seq ? p.max_seq : L);
  const int n = (L + p.split - 1) / p.split;
  uint8_t* o = (uint8_t*)p.out + ((int64_t)b * p.o_sb + (int64_t)hq * p.o_sh) * (p.out_bf16 ? 2 : 4);
  if (n == 0) {
    if (tid < 32) {
      if (p.out_bf16) *(u32x2*)(o + 8 * tid) = u32x2{0, 0};
      else *(f32x4*)(o + 16 * tid) = f32x4{0.f, 0.f, 0.f, 0.f};
    }
    return;
  }
  const int64_t slot0 = ((int64_t)b * p.num_q_heads + hq) * p.n_split;
  const int d4 = tid & 31, sg = tid >> 5;
  float M = -INFINITY, ls = 0.f;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  for (int c = sg; c < n; c += kMergeGroups * kMergeUnroll) {
    float mc[kMergeUnroll], lc[kMergeUnroll];
    f32x4 oc[kMergeUnroll];
#pragma unroll
    for (int u = 0; u < kMergeUnroll; ++u) {
      const int cc = c + u * kMergeGroups;
      if (cc < n) {
        const u32x2 ml = *(const u32x2*)(p.ws_ml + 2 * (slot0 + cc));
        mc[u] = __uint_as_float(ml[0]);
        lc[u] = __uint_as_float(ml[1]);
        oc[u] = *(const f32x4*)(p.ws_o + (slot0 + cc) * kHeadDim + 4 * d4);
      } else {
        mc[u] = -INFINITY;
        lc[u] = 0.f;
        oc[u] = f32x4{0.f, 0.f, 0.f, 0.f};
      }
    }
    float mb = M;
#pragma unroll
    for (int u = 0; u < kMergeUnroll; ++u) mb = fmaxf(mb, mc[u]);
    const float corr = fast_exp2(M - mb);   // 0 while M = -inf
    ls *= corr;
    acc *= corr;
#pragma unroll
    for (int u = 0; u < kMergeUnroll; ++u) {
      const float w = fast_exp2(mc[u] - mb);
      ls += w * lc[u];
      acc += w * oc[u];
    }
    M = mb;
  }
  *(f32x4*)&racc[sg][4 * d4] = acc;
  if (d4 == 0) {
    rm[sg] = M;
    rl[sg] = ls;
  }
  __syncthreads();
  if (tid < 32) {
    float Mt = rm[0];
#pragma unroll
    for (int j = 1; j < kMergeGroups; ++j) Mt = fmaxf(Mt, rm[j]);
    f32x4 t = {0.f, 0.f, 0.f, 0.f};
    float lt = 0.f;
#pragma unroll
    for (int j = 0; j < kMergeGroups; ++j) {
      const float w = fast_exp2(rm[j] - Mt);   // 0 for a group that held no chunk
      t += w * *(const f32x4*)&racc[j][4 * tid];
      lt += w * rl[j];
    }
    t *= 1.0f / lt;
    if (p.out_bf16) *(u32x2*)(o + 8 * tid) = u32x2{pack_bf16x2(t[0], t[1]), pack_bf16x2(t[2], t[3])};
    else *(f32x4*)(o + 16 * tid) = t;
  }
}

}  // namespace

hipError_t launch_decode_partition(const DecodeParams& p, bool in_bf16, hipStream_t stream) {
  const dim3 grid(p.n_split, p.num_kv_heads, p.batch);
  if (in_bf16) {
    hipLaunchKernelGGL(decode_partition_kernel<true>, grid, dim3(kThreads), 0, stream, p);
  } else {
    hipLaunchKernelGGL(decode_partition_kernel<false>, grid, dim3(kThreads), 0, stream, p);
  }
  return hipGetLastError();
}

hipError_t launch_decode_merge(const DecodeParams& p, hipStream_t stream) {
  if (p.n_split == 1) return hipSuccess;
  hipLaunchKernelGGL(decode_merge_kernel, dim3(p.num_q_heads, p.batch), dim3(kMergeThreads), 0, stream, p);
  return hipGetLastError();
}

}  // namespace gqa
