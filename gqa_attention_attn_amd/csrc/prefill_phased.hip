// Two-phase causal prefill for gfx950 (MI355X): the key prologue once per key
// row, then attention with the query prologue fused in.
//
// "Qwen3-14B Optimization", section 2.1 "Shape 4": rope / QK-norm and the
// attention are one fused stage whose rope phase and attention phase are
// separated by an in-kernel grid-wide barrier.  On the GPU the grid-wide
// barrier is the boundary between two dispatches on one stream:
//  * phase 1 (key_prologue_kernel): every key row of every (sequence, KV head)
//    goes through RMSNorm + RoPE once and is stored as bf16 K' in a workspace;
//  * phase 2 (attention_kernel): tiled online softmax ("ADR-0060: AHBM GQA
//    Fused Attention Kernel (Llama3-70B)", sections 3 and 5.4) over K' and V,
//    with each query row's prologue applied when the query tile is loaded.
// Compared with recomputing the key prologue for every (query block, key
// tile) pair, each key row is transformed once (about 32x less VALU work for
// a 4096-token causal prefill) at the cost of writing and re-reading K'.
//
// Attention mapping: a workgroup = (sequence, query head, 128-query block),
// 4 waves of 32 query rows, 64-key tiles double-buffered in LDS (K' rows with
// 16-byte chunks XOR-swizzled by key; V stored transposed with a key order that
// gives each lane its 8 keys as one 16-byte read); S^T = K' Q'^T and
// O^T = V^T P^T on v_mfma_f32_32x32x16_bf16; two workgroups per compute unit
// so one's softmax overlaps the other's matrix work; a 1-D grid ordered so a
// (sequence, KV head) group's workgroups share one XCD's L2, heaviest block
// first.
#include "common.hpp"

namespace gqa {
namespace {

constexpr int kXcds = 8;
constexpr int kAttnThreads = 256;
constexpr int kBM = 128;               // query rows per workgroup
constexpr int kBN = 64;                // keys per tile
constexpr int kVtRow = 72;             // V^T row stride in bf16 (64 keys + 8): conflict-free 16-byte reads
constexpr float kLazyRescale = 8.0f;   // rescale O only when a row max grows by more than 2^8

// ----------------------------------------------------------------- phase 1: key prologue

// 16 key rows per workgroup; a row is held by 16 lanes (dims 4c..4c+3 and
// 64+4c..64+4c+3), so RMSNorm reduces over 16 lanes and RoPE pairs (i, i+64)
// stay in one lane.
__global__ __launch_bounds__(256) void key_prologue_kernel(const PrefillParams p, uint16_t* kws) {
  __shared__ double inv_rev[kHeadDim / 2];
  const int b = blockIdx.z, h = blockIdx.y;
  const int tid = threadIdx.x, r = tid >> 4, c = tid & 15;
  const bool rope = p.rope_theta > 0.0;
  if (tid < 64 && rope) inv_rev[tid] = rope_inv_freq(tid, p.rope_log2_theta) * 0.15915494309189535;
  __syncthreads();
  int n = p.seq_lens[b];
  n = n < 0 ? 0 : (n > p.max_seq ? p.max_seq : n);
  const int key = blockIdx.x * 16 + r;
  if (key >= n) return;   // whole 16-lane groups leave together
  const uint16_t* src = (const uint16_t*)p.k + ((int64_t)b * p.k_sb + (int64_t)h * p.k_sh + (int64_t)key * p.k_ss);
  const u32x2 lo = *(const u32x2*)(src + 4 * c);
  const u32x2 hi = *(const u32x2*)(src + 64 + 4 * c);
  float x[8] = {bf16lo(lo[0]), bf16hi(lo[0]), bf16lo(lo[1]), bf16hi(lo[1]),
                bf16lo(hi[0]), bf16hi(hi[0]), bf16lo(hi[1]), bf16hi(hi[1])};
  if (p.k_norm_w) {
    float ss = 0.f;
#pragma unroll
    for (int j = 0; j < 8; ++j) ss += x[j] * x[j];
    ss = sum16(ss);
    const float rr = 1.0f / sqrtf(ss * (1.0f / kHeadDim) + p.eps);
    const uint16_t* g = (const uint16_t*)p.k_norm_w;
    const u32x2 glo = *(const u32x2*)(g + 4 * c), ghi = *(const u32x2*)(g + 64 + 4 * c);
    const float gv[8] = {bf16lo(glo[0]), bf16hi(glo[0]), bf16lo(glo[1]), bf16hi(glo[1]),
                         bf16lo(ghi[0]), bf16hi(ghi[0]), bf16lo(ghi[1]), bf16hi(ghi[1])};
#pragma unroll
    for (int j = 0; j < 8; ++j) x[j] *= rr * gv[j];
  }
  if (rope) {
    const double kpos = (double)p.positions[b] + (double)key;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      float cs, sn;
      rope_cos_sin_rev(kpos, inv_rev[4 * c + j], cs, sn);
      const float a = x[j], bb = x[4 + j];
      x[j] = a * cs - bb * sn;
      x[4 + j] = bb * cs + a * sn;
    }
  }
  uint16_t* dst = kws + (((int64_t)b * p.num_kv_heads + h) * p.max_seq + key) * kHeadDim;
  *(u32x2*)(dst + 4 * c) = u32x2{pack_bf16x2(x[0], x[1]), pack_bf16x2(x[2], x[3])};
  *(u32x2*)(dst + 64 + 4 * c) = u32x2{pack_bf16x2(x[4], x[5]), pack_bf16x2(x[6], x[7])};
}

// ----------------------------------------------------------------- phase 2: attention

// Logical 16-byte chunk (of 16 per 128-dim row) holding QK operand slot kk of
// lane half hf: the lane's slots cover dims [32hf, 32hf+32) and
// [64+32hf, 64+32hf+32), so every query RoPE pair (i, i+64) stays in one lane.
__device__ __forceinline__ int qk_chunk(int kk, int hf) { return kk < 4 ? 4 * hf + kk : 8 + 4 * hf + (kk - 4); }

// K' chunk swizzle: a bijection on keys mod 16 (conflict-free operand reads of
// 16 consecutive keys) alternating the 128-byte half between neighbouring keys.
__device__ __forceinline__ int kswz(int key) { return (key & 15) ^ ((key & 1) << 3); }

// Position of key k (0..63) of a tile in a V^T row: key 32u + 16e + 8a + 4h + r
// goes to 32u + 16e + 8h + 4a + r, so the 8 keys that PV MFMA (u, e) of lane
// half h takes are 16 contiguous bytes.
__device__ __forceinline__ int vpos(int k) { return (k & 0x33) | ((k & 4) << 1) | ((k & 8) >> 1); }

struct __attribute__((aligned(16))) AttnSmem {
  uint32_t kt[2][kBN][kHeadDim / 2];   // K' tiles (bf16 pairs), swizzled 16-byte chunks
  uint16_t vt[2][kHeadDim][kVtRow];    // V^T tiles: vt[buf][dim][vpos(key)]
  double inv_rev[kHeadDim / 2];        // query RoPE: theta^(-2i/128) / (2 pi)
};

// Staging of one 64-key tile, one unit per thread:
//  K': key row t/4, logical chunks 4(t%4) .. 4(t%4)+3 (64 bytes);
//  V : key rows 2(t%32), 2(t%32)+1, dims 16(t/32) .. +15 (2 x 32 bytes).
struct TileRegs { u32x4 k[4]; u32x4 v[4]; };

struct Slabs {
  const uint8_t* kb;   // K' rows of this (sequence, KV head), 256 bytes each
  const uint8_t* vb;
  uint32_t vss;        // V row stride in bytes
  int n;
};

__device__ __forceinline__ void fetch_tile(TileRegs& t, const Slabs& s, int kt, int tid) {
  const int kkey = kt * kBN + (tid >> 2);
  if (kkey < s.n) {
    const u32x4* src = (const u32x4*)(s.kb + (uint32_t)kkey * 256u + 64u * (tid & 3));
#pragma unroll
    for (int j = 0; j < 4; ++j) t.k[j] = src[j];
  } else {
#pragma unroll
    for (int j = 0; j < 4; ++j) t.k[j] = u32x4{0, 0, 0, 0};
  }
  const int vkey = kt * kBN + 2 * (tid & 31), dc = tid >> 5;
  const uint8_t* v0 = s.vb + (uint32_t)vkey * s.vss + 32u * dc;
  if (vkey < s.n) {
    t.v[0] = *(const u32x4*)v0;
    t.v[1] = *(const u32x4*)(v0 + 16);
  } else {
    t.v[0] = t.v[1] = u32x4{0, 0, 0, 0};
  }
  if (vkey + 1 < s.n) {
    t.v[2] = *(const u32x4*)(v0 + s.vss);
    t.v[3] = *(const u32x4*)(v0 + s.vss + 16);
  } else {
    t.v[2] = t.v[3] = u32x4{0, 0, 0, 0};
  }
}

__device__ __forceinline__ void stage_tile(AttnSmem& sm, const TileRegs& t, int buf, int tid) {
  const int kkey = tid >> 2, c0 = 4 * (tid & 3);
  uint32_t* krow = sm.kt[buf][kkey];
  const int sw = kswz(kkey);
#pragma unroll
  for (int j = 0; j < 4; ++j) *(u32x4*)(krow + 4 * ((c0 + j) ^ sw)) = t.k[j];
  const int kp = tid & 31, dc = tid >> 5;
  const int pos = vpos(2 * kp);   // keys 2kp, 2kp+1 stay adjacent
#pragma unroll
  for (int j = 0; j < 8; ++j) {   // dims 16dc + 2j, 16dc + 2j + 1
    const uint32_t a = t.v[j >> 2][j & 3], bb = t.v[2 + (j >> 2)][j & 3];
    *(uint32_t*)&sm.vt[buf][16 * dc + 2 * j][pos] = pair_lo(a, bb);
    *(uint32_t*)&sm.vt[buf][16 * dc + 2 * j + 1][pos] = pair_hi(a, bb);
  }
}

__global__ __launch_bounds__(kAttnThreads, 2) void attention_kernel(const PrefillParams p, const uint16_t* kws) {
  __shared__ AttnSmem sm;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int n32 = lane & 31, hf = lane >> 5;
  const int G = p.group;

  // ---- workgroup -> (sequence, KV head group, query head, 128-query block)
  const int nqb = p.n_qblocks;
  const int per_group = nqb * G;
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
  const int qb = nqb - 1 - w / G;   // heaviest block first
  const int hq = h * G + w % G;

  int n = p.seq_lens[b];
  n = n < 0 ? 0 : (n > p.max_seq ? p.max_seq : n);
  const int q0 = qb * kBM;
  if (q0 >= n) return;
  const int qe = min(q0 + kBM, n);
  const int kend = p.causal ? qe : n;
  const int ntiles = (kend + kBN - 1) / kBN;
  const bool rope = p.rope_theta > 0.0;
  const double pos0 = (double)p.positions[b];
  const int wq0 = q0 + 32 * wave;
  const int qrow = wq0 + n32;
  const bool wave_live = wq0 < n;

  Slabs sl;
  sl.kb = (const uint8_t*)(kws + ((int64_t)b * p.num_kv_heads + h) * p.max_seq * kHeadDim);
  sl.vb = (const uint8_t*)p.v + ((int64_t)b * p.v_sb + (int64_t)h * p.v_sh) * 2;
  sl.vss = (uint32_t)(p.v_ss * 2);
  sl.n = n;

  TileRegs tr;
  fetch_tile(tr, sl, 0, tid);
  if (tid < 64 && rope) sm.inv_rev[tid] = rope_inv_freq(tid, p.rope_log2_theta) * 0.15915494309189535;

  // ---- query prologue: lane (n32, hf) owns row qrow of head hq, dims [32hf, 32hf+32) and [64+32hf, 64+32hf+32)
  bf16x8 qf[8];
  {
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
    stage_tile(sm, tr, 0, tid);
    if (ntiles > 1) fetch_tile(tr, sl, 1, tid);
    __syncthreads();   // tables and tile 0
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
      qf[j] = as_bf16x8(u32x4{pack_bf16x2(xl[0], xl[1]), pack_bf16x2(xl[2], xl[3]), pack_bf16x2(xl[4], xl[5]),
                              pack_bf16x2(xl[6], xl[7])});
      qf[4 + j] = as_bf16x8(u32x4{pack_bf16x2(xh[0], xh[1]), pack_bf16x2(xh[2], xh[3]), pack_bf16x2(xh[4], xh[5]),
                                  pack_bf16x2(xh[6], xh[7])});
    }
  }

  f32x16 o[4];
#pragma unroll
  for (int T = 0; T < 4; ++T)
#pragma unroll
    for (int i = 0; i < 16; ++i) o[T][i] = 0.f;
  float m_run = -INFINITY, l_run = 0.f;

  for (int kt = 0; kt < ntiles; ++kt) {
    const int buf = kt & 1;
    const int ks = kt * kBN;
    const bool future = p.causal && ks > wq0 + 31;
    if (wave_live && !future) {
      // sacc[u][i] = S[key ks + 32u + 8(i/4) + 4hf + i%4][query qrow] (raw)
      f32x16 sacc[2];
#pragma unroll
      for (int u = 0; u < 2; ++u) {
#pragma unroll
        for (int i = 0; i < 16; ++i) sacc[u][i] = 0.f;
        const int krow = 32 * u + n32;
        const uint32_t* kr = sm.kt[buf][krow];
        const int sw = kswz(krow);
#pragma unroll
        for (int kk = 0; kk < 8; ++kk) {
          const u32x4 a = *(const u32x4*)(kr + 4 * (qk_chunk(kk, hf) ^ sw));
          sacc[u] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(a), qf[kk], sacc[u], 0, 0, 0);
        }
      }
      if ((p.causal && ks + kBN - 1 > wq0) || ks + kBN > n) {   // wave-uniform: diagonal or ragged tile
        const int lim = (p.causal ? min(n, qrow + 1) : n) - ks - 4 * hf;
#pragma unroll
        for (int u = 0; u < 2; ++u)
#pragma unroll
          for (int i = 0; i < 16; ++i)
            sacc[u][i] = (32 * u + 8 * (i >> 2) + (i & 3) < lim) ? sacc[u][i] : -INFINITY;
      }
      float mx = fmaxf(sacc[0][0], sacc[1][0]);
#pragma unroll
      for (int i = 1; i < 16; ++i) mx = fmaxf(mx, fmaxf(sacc[0][i], sacc[1][i]));
      mx = max_xor32(mx) * p.scale_log2;
      if (__any(mx > m_run + kLazyRescale)) {   // lazy rescale (the final O / l is unaffected)
        const float m_new = fmaxf(m_run, mx);
        const float corr = fast_exp2(m_run - m_new);
        l_run *= corr;
#pragma unroll
        for (int T = 0; T < 4; ++T) o[T] *= corr;
        m_run = m_new;
      }
      float ps = 0.f;
#pragma unroll
      for (int u = 0; u < 2; ++u)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const float e = fast_exp2(fmaf(sacc[u][i], p.scale_log2, -m_run));
          sacc[u][i] = e;
          ps += e;
        }
      l_run += ps;
      // O^T += V^T P^T: MFMA (u, e) takes keys ks + 32u + 16e + {4hf + t, 8 + 4hf + t}, t < 4,
      // stored contiguously at V^T positions 32u + 16e + 8hf .. +7
#pragma unroll
      for (int u = 0; u < 2; ++u)
#pragma unroll
        for (int e = 0; e < 2; ++e) {
          const u32x4 pf = {pack_bf16x2(sacc[u][8 * e + 0], sacc[u][8 * e + 1]),
                            pack_bf16x2(sacc[u][8 * e + 2], sacc[u][8 * e + 3]),
                            pack_bf16x2(sacc[u][8 * e + 4], sacc[u][8 * e + 5]),
                            pack_bf16x2(sacc[u][8 * e + 6], sacc[u][8 * e + 7])};
#pragma unroll
          for (int T = 0; T < 4; ++T) {
            const u32x4 a = *(const u32x4*)&sm.vt[buf][32 * T + n32][32 * u + 16 * e + 8 * hf];
            o[T] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(a), as_bf16x8(pf), o[T], 0, 0, 0);
          }
        }
    }
    // ---- stage tile kt+1 (other buffer, unread since the last barrier), fetch kt+2
    if (kt + 1 < ntiles) {
      stage_tile(sm, tr, buf ^ 1, tid);
      if (kt + 2 < ntiles) fetch_tile(tr, sl, kt + 2, tid);
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

size_t prefill_workspace_bytes(int batch, int num_kv_heads, int max_seq) {
  return (size_t)batch * num_kv_heads * max_seq * kHeadDim * 2;
}

hipError_t launch_prefill_phased(const PrefillParams& p, void* workspace, hipStream_t stream) {
  uint16_t* kws = (uint16_t*)workspace;
  hipLaunchKernelGGL(key_prologue_kernel, dim3((p.max_seq + 15) / 16, p.num_kv_heads, p.batch), dim3(256), 0, stream, p,
                     kws);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  PrefillParams q = p;
  q.n_qblocks = (p.max_seq + kBM - 1) / kBM;
  hipLaunchKernelGGL(attention_kernel, dim3(q.n_qblocks * p.num_q_heads * p.batch), dim3(kAttnThreads), 0, stream, q,
                     (const uint16_t*)kws);
  return hipGetLastError();
}

}  // namespace gqa
