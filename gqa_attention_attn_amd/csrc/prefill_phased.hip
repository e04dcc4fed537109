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
// Attention mapping: a workgroup = (sequence, query head, 128-query block) of
// 4 waves x 32 query rows, two workgroups per compute unit; 64-key tiles
// filled by direct-to-LDS loads (no register staging): K' rows at a padded
// pitch, V in natural [key][dim] rows read back transposed by
// ds_read_b64_tr_b16 as the V^T operand; S^T = K' Q'^T and O^T = V^T P^T on
// v_mfma_f32_32x32x16_bf16.  Software pipeline: the scores of tile t+1 are
// computed while the softmax of tile t runs; K' is loaded two tiles ahead and
// V one tile ahead, so one barrier per tile suffices.  A 1-D grid ordered so a
// (sequence, KV head) group's workgroups share one XCD's L2, heaviest block
// first.
#include "common.hpp"

namespace gqa {
namespace {

constexpr int kXcds = 8;
constexpr int kAttnThreads = 256;      // 4 waves of 32 query rows
constexpr int kBM = 128;               // query rows per workgroup
constexpr int kBN = 64;                // keys per tile
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

// LDS tiles of 64 keys, double-buffered.  K' rows are 256 bytes at a 272-byte
// pitch (16 consecutive rows read 16 bytes each on distinct banks), V rows
// (natural [key][dim] order) 256 bytes at a 288-byte pitch (the transposing
// reads of 4 consecutive rows x 32 bytes hit distinct banks).  Every operand
// read is then one lane base address plus an immediate offset.
constexpr int kKPitch = 272;
constexpr int kVPitch = 288;
constexpr int kKTileBytes = kBN * kKPitch;   // 17 KiB: 17 direct-to-LDS loads of 1 KiB
constexpr int kVTileBytes = kBN * kVPitch;   // 18 KiB: 18 loads

#define LDS_AS __attribute__((address_space(3)))

// One 1 KiB direct-to-LDS load: lane l's 16 bytes from `src` land at LDS
// bytes lds + 16 l.  Issued from inline assembly so that the compiler does not
// wait for it before unrelated LDS reads; completion is waited for explicitly
// (s_waitcnt vmcnt) before the barrier that publishes the tile.  M0 carries
// the LDS address; nothing else in these kernels uses M0.
__device__ __forceinline__ void dma16(uint32_t lds, const void* src) {
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
  asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, off" ::"s"(lds), "v"(src) : "memory", "m0");
#pragma clang diagnostic pop
}

// Fill of one tile: LDS byte A = 1024 i + 16 l of the tile is row A / pitch,
// 16-byte chunk (A % pitch) / 16; chunks past the 16 of a row are padding and
// take a copy of chunk 15.  Wave w issues loads i = w, w + 4, ...; DmaLane
// holds the row and source byte offset of each of them for this lane.  Rows
// at or past n read row n-1 (valid data; their scores are masked and their P
// is zero).
template <int PITCH>
struct DmaLane {
  static constexpr int kCh = PITCH / 16;            // 17 or 18 chunks per row
  static constexpr int kLoads = kBN * kCh / 64;     // 17 or 18 loads per tile
  static constexpr int kPerWave = (kLoads + 3) / 4; // at most 5 per wave
  int row[kPerWave];
  uint32_t off[kPerWave];                           // row * stride + 16 * chunk
  __device__ __forceinline__ void init(uint32_t row_stride, int wave, int lane) {
#pragma unroll
    for (int m = 0; m < kPerWave; ++m) {
      const int a = 64 * (wave + 4 * m) + lane;
      const int r = a / kCh, ch = min(a - r * kCh, 15);
      row[m] = r;
      off[m] = (uint32_t)r * row_stride + 16u * ch;
    }
  }
};

template <int PITCH>
__device__ __forceinline__ void dma_tile(uint32_t lds, const uint8_t* slab, uint32_t row_stride, const DmaLane<PITCH>& dl,
                                         int key0, int n, int wave) {
  constexpr int kLoads = DmaLane<PITCH>::kLoads;
  const uint8_t* base = slab + (uint32_t)key0 * row_stride;
  if (key0 + kBN <= n) {   // wave-uniform: every row of the tile is valid
#pragma unroll
    for (int m = 0; m < DmaLane<PITCH>::kPerWave; ++m)
      if (wave + 4 * m < kLoads) dma16(lds + 1024u * (wave + 4 * m), base + dl.off[m]);
  } else {
#pragma unroll
    for (int m = 0; m < DmaLane<PITCH>::kPerWave; ++m) {
      if (wave + 4 * m >= kLoads) continue;
      const int over = key0 + dl.row[m] - (n - 1);   // rows past n-1 move back to n-1
      const uint32_t off = over > 0 ? dl.off[m] - (uint32_t)over * row_stride : dl.off[m];
      dma16(lds + 1024u * (wave + 4 * m), base + off);
    }
  }
}

// S^T for the 64 keys of a K' tile and the wave's 32 query rows:
// s[kb][i] = S[key 32kb + 8(i/4) + 4hf + i%4][query n32] (raw dot products).
__device__ __forceinline__ void qk_tile(f32x16 (&s)[2], const LDS_AS uint8_t* kt, const bf16x8 (&qf)[8], int n32,
                                        int hf) {
  const LDS_AS uint8_t* base = kt + kKPitch * n32 + 64 * hf;
#pragma unroll
  for (int kb = 0; kb < 2; ++kb)
#pragma unroll
    for (int i = 0; i < 16; ++i) s[kb][i] = 0.f;
#pragma unroll
  for (int kk = 0; kk < 8; ++kk)
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      const u32x4 a = *(const LDS_AS u32x4*)(base + kKPitch * 32 * kb + 16 * ((kk & 3) + 8 * (kk >> 2)));
      s[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(a), qf[kk], s[kb], 0, 0, 0);
    }
}

// Online softmax of one tile in two parts (log2 units, lazy rescale):
// softmax_max masks, takes the row maximum and rescales O when it grew by
// more than 2^8; softmax_exp forms P and leaves P^T as bf16 MFMA operands
// pf[u][e] (keys 32u + 16e + {4hf+t, 8+4hf+t}, t < 4).  The scores of the
// next tile are computed between the two so that they share a basic block
// with the exponentials.
struct RowState { float m, l; };

// IEEE maximum (NaN-propagating) needs no quieting of its MFMA-produced
// operands, and pairs of it fuse into v_maximum3: 17 instructions for the
// 32 scores a lane holds.
__device__ __forceinline__ float max3(float a, float b, float c) {
  return __builtin_elementwise_maximum(__builtin_elementwise_maximum(a, b), c);
}

__device__ __forceinline__ float row_max32(const f32x16 (&s)[2]) {
  float t[11];
#pragma unroll
  for (int u = 0; u < 2; ++u)
#pragma unroll
    for (int i = 0; i < 5; ++i) t[5 * u + i] = max3(s[u][3 * i], s[u][3 * i + 1], s[u][3 * i + 2]);
  t[10] = __builtin_elementwise_maximum(s[0][15], s[1][15]);
  return max3(max3(t[0], t[1], t[2]), max3(t[3], t[4], t[5]),
              max3(t[6], t[7], __builtin_elementwise_maximum(t[8], __builtin_elementwise_maximum(t[9], t[10]))));
}

__device__ __forceinline__ void softmax_max(f32x16 (&s)[2], RowState& st, f32x16 (&o)[4], bool mask, int lim,
                                            float scale_log2) {
  if (mask) {   // keys at tile offsets >= lim (this lane's half) are invisible
#pragma unroll
    for (int u = 0; u < 2; ++u)
#pragma unroll
      for (int i = 0; i < 16; ++i) s[u][i] = (32 * u + 8 * (i >> 2) + (i & 3) < lim) ? s[u][i] : -INFINITY;
  }
  float mx = row_max32(s);
  mx = max_xor32(mx) * scale_log2;
  if (__any(mx > st.m + kLazyRescale)) {   // lazy rescale (the final O / l is unaffected)
    const float m_new = fmaxf(st.m, mx);
    const float corr = fast_exp2(st.m - m_new);
    st.l *= corr;
#pragma unroll
    for (int T = 0; T < 4; ++T) o[T] *= corr;
    st.m = m_new;
  }
}

// The row sum l is taken over the bf16-rounded P that the P V products use
// (v_dot2 of each packed pair with (1, 1)), so numerator and denominator see
// the same weights.
__device__ __forceinline__ void softmax_exp(f32x16 (&s)[2], RowState& st, u32x4 (&pf)[2][2], float scale_log2) {
#pragma unroll
  for (int u = 0; u < 2; ++u)
#pragma unroll
    for (int i = 0; i < 16; ++i) s[u][i] = fast_exp2(fmaf(s[u][i], scale_log2, -st.m));
#pragma unroll
  for (int u = 0; u < 2; ++u)
#pragma unroll
    for (int e = 0; e < 2; ++e)
      pf[u][e] = u32x4{pack_bf16x2(s[u][8 * e + 0], s[u][8 * e + 1]), pack_bf16x2(s[u][8 * e + 2], s[u][8 * e + 3]),
                       pack_bf16x2(s[u][8 * e + 4], s[u][8 * e + 5]), pack_bf16x2(s[u][8 * e + 6], s[u][8 * e + 7])};
  const bf16x2 one = {(__bf16)1.0f, (__bf16)1.0f};
  float ps[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int u = 0; u < 2; ++u)
#pragma unroll
    for (int e = 0; e < 2; ++e)
#pragma unroll
      for (int w = 0; w < 4; ++w)   // the (uint32_t) copy matters: hipcc bit-casts element 0 of a vector lvalue
        ps[w] = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, (uint32_t)pf[u][e][w]), one, ps[w], false);
  st.l += (ps[0] + ps[1]) + (ps[2] + ps[3]);
}

// O^T += V^T P^T.  The V^T operand of MFMA (u, e), dim tile T comes from two
// transposing reads of natural V rows: lane group g (16 lanes) covers dims
// 32T + 16(g%2) .. +15 and keys R = 32u + 16e + 8a + 4(g/2) .. R+3 for
// a = 0, 1 (slots 4a .. 4a+3); source lane j of the group points at key
// R + j/4, dims + 4(j%4) .. +3.
typedef __attribute__((__vector_size__(4 * sizeof(__bf16)))) __bf16 bf16x4_v;

__device__ __forceinline__ void pv_tile(f32x16 (&o)[4], const LDS_AS uint8_t* vt, const u32x4 (&pf)[2][2], int lane) {
  const int g = lane >> 4, j = lane & 15;
  const LDS_AS uint8_t* base = vt + kVPitch * (4 * (g >> 1) + (j >> 2)) + 2 * (16 * (g & 1) + 4 * (j & 3));
#pragma unroll
  for (int u = 0; u < 2; ++u)
#pragma unroll
    for (int e = 0; e < 2; ++e)
#pragma unroll
      for (int T = 0; T < 4; ++T) {
        const bf16x4_v x0 = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
            (LDS_AS bf16x4_v*)(base + kVPitch * (32 * u + 16 * e) + 64 * T));
        const bf16x4_v x1 = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
            (LDS_AS bf16x4_v*)(base + kVPitch * (32 * u + 16 * e + 8) + 64 * T));
        const bf16x8 a = __builtin_shufflevector(x0, x1, 0, 1, 2, 3, 4, 5, 6, 7);
        o[T] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, as_bf16x8(pf[u][e]), o[T], 0, 0, 0);
      }
}

struct WaveCtx {
  int qrow;       // this lane's query row
  int wq0;        // first query row of the wave
  int n;          // sequence length
  bool causal;
  float scale_log2;
};

// Tile t of the wave: softmax of s_cur (tile t) and P V from vt (V_t);
// s_next receives the scores of the tile in kt_next (tile t+1; on the wave's
// last tile the products are computed and discarded, which keeps the matrix
// work in the same basic block as the exponentials it overlaps).
__device__ __forceinline__ void wave_tile(int t, f32x16 (&s_cur)[2], f32x16 (&s_next)[2],
                                          const LDS_AS uint8_t* kt_next, const LDS_AS uint8_t* vt,
                                          const bf16x8 (&qf)[8], f32x16 (&o)[4], RowState& st, const WaveCtx& w,
                                          int lane) {
  const int n32 = lane & 31, hf = lane >> 5;
  const int ks = t * kBN;
  const bool mask = (w.causal && ks + kBN - 1 > w.wq0) || ks + kBN > w.n;   // wave-uniform
  const int lim = (w.causal ? min(w.n, w.qrow + 1) : w.n) - ks - 4 * hf;
  softmax_max(s_cur, st, o, mask, lim, w.scale_log2);
  qk_tile(s_next, kt_next, qf, n32, hf);
  u32x4 pf[2][2];
  softmax_exp(s_cur, st, pf, w.scale_log2);
  pv_tile(o, vt, pf, lane);
}

// Workgroup: 4 waves x 32 query rows of one query head, 64-key tiles, two
// workgroups per compute unit.  Pipeline per tile t (one barrier): at the
// start of step t the loads of K'_{t+2} (into the buffer of K'_t, whose scores
// were computed in step t-1) and of V_{t+1} (into the buffer of V_{t-1}) are
// issued; step t computes the scores of tile t+1 and the softmax and P V of
// tile t; the loads are waited for before the closing barrier.
__global__ __launch_bounds__(kAttnThreads, 2) void attention_kernel(const PrefillParams p, const uint16_t* kws) {
  __shared__ __attribute__((aligned(16))) uint8_t kt0[kKTileBytes], kt1[kKTileBytes];
  __shared__ __attribute__((aligned(16))) uint8_t vt0[kVTileBytes], vt1[kVTileBytes];
  __shared__ double inv_rev[kHeadDim / 2];   // query RoPE: theta^(-2i/128) / (2 pi)
  LDS_AS uint8_t* const K0 = (LDS_AS uint8_t*)kt0;
  LDS_AS uint8_t* const K1 = (LDS_AS uint8_t*)kt1;
  LDS_AS uint8_t* const V0 = (LDS_AS uint8_t*)vt0;
  LDS_AS uint8_t* const V1 = (LDS_AS uint8_t*)vt1;
  const uint32_t k0a = (uint32_t)(uintptr_t)K0, k1a = (uint32_t)(uintptr_t)K1;
  const uint32_t v0a = (uint32_t)(uintptr_t)V0, v1a = (uint32_t)(uintptr_t)V1;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
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

  WaveCtx wc;
  wc.wq0 = q0 + 32 * wave;
  wc.qrow = wc.wq0 + n32;
  wc.n = n;
  wc.causal = p.causal != 0;
  wc.scale_log2 = p.scale_log2;
  const bool wave_live = wc.wq0 < n;
  const int wkend = !wave_live ? 0 : (wc.causal ? min(n, wc.wq0 + 32) : n);
  const int wtiles = (wkend + kBN - 1) / kBN;   // tiles 0 .. wtiles-1 hold keys this wave sees

  const uint8_t* kslab = (const uint8_t*)(kws + ((int64_t)b * p.num_kv_heads + h) * p.max_seq * kHeadDim);
  const uint8_t* vslab = (const uint8_t*)p.v + ((int64_t)b * p.v_sb + (int64_t)h * p.v_sh) * 2;
  const uint32_t vss = (uint32_t)(p.v_ss * 2);

  // ---- first tiles requested before the query prologue
  DmaLane<kKPitch> dk;
  DmaLane<kVPitch> dv;
  dk.init(256u, wave, lane);
  dv.init(vss, wave, lane);
  dma_tile<kKPitch>(k0a, kslab, 256u, dk, 0, n, wave);
  dma_tile<kVPitch>(v0a, vslab, vss, dv, 0, n, wave);
  if (ntiles > 1) dma_tile<kKPitch>(k1a, kslab, 256u, dk, kBN, n, wave);
  if (tid < 64 && rope) inv_rev[tid] = rope_inv_freq(tid, p.rope_log2_theta) * 0.15915494309189535;

  // ---- query prologue: lane (n32, hf) owns row wq0 + n32 of head hq,
  //      dims [32hf, 32hf+32) and [64+32hf, 64+32hf+32)
  bf16x8 qf[8];
  {
    u32x4 qlo[4], qhi[4];
    if (wc.qrow < n) {
      const uint16_t* row = (const uint16_t*)p.q + ((int64_t)b * p.q_sb + (int64_t)hq * p.q_sh + (int64_t)wc.qrow * p.q_ss);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        qlo[j] = *(const u32x4*)(row + 32 * hf + 8 * j);
        qhi[j] = *(const u32x4*)(row + 64 + 32 * hf + 8 * j);
      }
    } else {
#pragma unroll
      for (int j = 0; j < 4; ++j) qlo[j] = qhi[j] = u32x4{0, 0, 0, 0};
    }
    __builtin_amdgcn_s_waitcnt(0);   // this thread's tile loads (and q row) have landed
    __syncthreads();                 // tables, K'_0, K'_1, V_0
    const uint16_t* g = (const uint16_t*)p.q_norm_w;
    float r = 1.0f;
    if (g) {
      float ss = 0.f;
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float a = bf16_elem(qlo[j], e), c = bf16_elem(qhi[j], e);
          ss += a * a + c * c;
        }
      ss = sum_xor32(ss);
      r = rsqrtf(ss * (1.0f / kHeadDim) + p.eps);
    }
    const double qpos = pos0 + (double)wc.qrow;
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
          rope_cos_sin_rev(qpos, inv_rev[32 * hf + 8 * j + e], c, s);
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
  RowState st = {-INFINITY, 0.f};

  f32x16 sa[2], sb[2];
  if (wtiles > 0) qk_tile(sa, K0, qf, n32, hf);
  __syncthreads();   // every read of K'_0 done: its buffer takes K'_2

  // two tiles per trip: buffers and score registers have fixed roles in each half
  for (int t = 0; t < ntiles; t += 2) {
    if (t + 2 < ntiles) dma_tile<kKPitch>(k0a, kslab, 256u, dk, (t + 2) * kBN, n, wave);
    if (t + 1 < ntiles) dma_tile<kVPitch>(v1a, vslab, vss, dv, (t + 1) * kBN, n, wave);
    if (t < wtiles) wave_tile(t, sa, sb, K1, V0, qf, o, st, wc, lane);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    const int t1 = t + 1;
    if (t1 >= ntiles) break;
    if (t1 + 2 < ntiles) dma_tile<kKPitch>(k1a, kslab, 256u, dk, (t1 + 2) * kBN, n, wave);
    if (t1 + 1 < ntiles) dma_tile<kVPitch>(v0a, vslab, vss, dv, (t1 + 1) * kBN, n, wave);
    if (t1 < wtiles) wave_tile(t1, sb, sa, K0, V1, qf, o, st, wc, lane);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
  }

  // ---- epilogue: O / l for this lane's query row
  if (!wave_live) return;
  const float l = sum_xor32(st.l);
  if (wc.qrow >= n) return;
  const float inv = 1.0f / l;
  uint8_t* orow = (uint8_t*)p.out + ((int64_t)b * p.o_sb + (int64_t)hq * p.o_sh + (int64_t)wc.qrow * p.o_ss) * (p.out_bf16 ? 2 : 4);
  // o[T][4a + r] = O[query][dim 32T + 8a + 4hf + r]
#pragma unroll
  for (int T = 0; T < 4; ++T) {
#pragma unroll
    for (int a = 0; a < 4; ++a) {
      const int d0 = 32 * T + 8 * a + 4 * hf;
      const float v0 = o[T][4 * a] * inv, v1 = o[T][4 * a + 1] * inv;
      const float v2 = o[T][4 * a + 2] * inv, v3 = o[T][4 * a + 3] * inv;
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
