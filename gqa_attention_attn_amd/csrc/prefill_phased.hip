// Two-phase causal prefill for gfx950 (MI355X): the key prologue once per key
// row, then attention with the query prologue fused in.
//
// "Qwen3-14B Optimization", section 2.1 "Shape 4": rope / QK-norm and the
// attention are one fused stage whose rope phase and attention phase are
// separated by an in-kernel grid-wide barrier.  On the GPU the grid-wide
// barrier is the boundary between two dispatches on one stream:
//  * phase 1 (key_prologue_kernel): every key row of every (sequence, KV head)
//    goes through RMSNorm + RoPE once and is stored as fp16 K' in a workspace,
//    beside its V row converted to fp16, both already in the padded row
//    layout the attention tiles have in LDS;
//  * phase 2 (attention_kernel): tiled online softmax ("ADR-0060: AHBM GQA
//    Fused Attention Kernel (Llama3-70B)", sections 3 and 5.4) over K' and V,
//    with each query row's prologue applied when the query tile is loaded.
// Compared with recomputing the key prologue for every (query block, key
// tile) pair, each key row is transformed once (about 32x less VALU work for
// a 4096-token causal prefill) at the cost of writing and re-reading K' and V.
//
// Attention mapping: a workgroup = (sequence, query head, 128-query block,
// key span) of 4 waves x 32 query rows, three waves per SIMD (three
// workgroups per compute unit).  32-key tiles are filled by linear direct-to-LDS copies (no register
// staging) from the padded workspace; V is read back transposed by
// ds_read_b64_tr_b16 as the V^T operand.  S^T = K' Q'^T and O^T = V^T P^T run
// on v_mfma_f32_32x32x16_f16 (the bf16 rate, with 11 significand bits for
// the rounded q', k' and P instead of 8; bf16 V converts to fp16 exactly for
// magnitudes in [2^-14, 65504]).  Software pipeline of a wave, per tile t: the
// scores of tile t+1 are computed beside the exponentials of tile t, then P V
// of tile t, then the row maxima of tile t+1; K' is loaded two tiles ahead
// and V one tile ahead, so one barrier per tile suffices.  A 1-D grid ordered
// so a (sequence, KV head) group's workgroups share one XCD's L2, largest
// item first; when the grid is short, the key range of a long query block is
// split over several workgroups whose states are merged by the last of them.
#include <algorithm>
#include <utility>
#include <vector>

#include "common.hpp"
#ifdef GQA_TIMELINE
#include "gqa_timeline.h"
#endif

namespace gqa {
namespace {

constexpr int kXcds = 8;
constexpr int kBM = 128;                 // query rows per workgroup
// 32-row MFMA blocks per wave.  Two blocks per wave would share every K' and
// V operand read from LDS (half the LDS traffic per product), but their
// registers leave one wave per SIMD, whose in-order issue serialises the
// matrix and vector work; one block per wave with three waves per SIMD is
// faster.
constexpr int kRB = 1;
constexpr int kWaves = kBM / (32 * kRB);  // waves per workgroup
// Per-workgroup timeline of the attention kernel, compiled in only with
// -DGQA_TIMELINE (the measurement build; include/gqa_timeline.h lists the
// stamps): thread 0 takes s_memrealtime stamps into LDS, the workgroup writes
// them out after its tile loop, and thread 0 stores its end stamp at its exit.
// Without the flag the stamp sites expand to nothing.
#ifdef GQA_TIMELINE
__device__ uint64_t g_timeline_attn[GQA_TIMELINE_BLOCKS * GQA_TIMELINE_SLOTS];
#define GQA_STAMP(i)                                            \
  do {                                                          \
    if (tid == 0) tla[(i)] = __builtin_amdgcn_s_memrealtime();  \
  } while (0)
#define GQA_STAMP_END()                                                                                   \
  do {                                                                                                    \
    if (tid == 0 && blockIdx.x < GQA_TIMELINE_BLOCKS)                                                     \
      g_timeline_attn[blockIdx.x * GQA_TIMELINE_SLOTS + 5] = __builtin_amdgcn_s_memrealtime();            \
  } while (0)
#else
#define GQA_STAMP(i)
#define GQA_STAMP_END()
#endif
constexpr int kWavesPerSimd = 3;   // 168 VGPRs; the tile loop holds no spill (the span merge does)
constexpr int kAttnThreads = 64 * kWaves;
constexpr int kBN = 32;                  // keys per tile
constexpr float kLazyRescale = 8.0f;     // rescale O only when a row max grows by more than 2^8

// Workspace: per (sequence, KV head), tiles of 32 keys, each 9 KiB: K' rows
// of 256 bytes at a 272-byte pitch (8.5 KiB, the rest slack) and V rows of
// 256 bytes at a 288-byte pitch, in separate regions; padding bytes are never
// written nor read.  max_seq is rounded up to whole tiles; rows in
// [n, round_up(n, 32)) hold zeros.  A tile is copied to LDS as is: there 16
// consecutive K' rows read 16 bytes each on distinct banks, and the
// transposing V reads of 4 consecutive rows x 32 bytes hit distinct banks.
constexpr int kKPitch = 272;
constexpr int kVPitch = 288;
constexpr int kTileBytes = 9216;             // 9 direct-to-LDS copies of 1 KiB
static_assert(kBN * kKPitch <= kTileBytes && kBN * kVPitch == kTileBytes, "tile layout");

__host__ __device__ inline int64_t ws_tiles(int max_seq) { return ((int64_t)max_seq + kBN - 1) / kBN; }

// Extent of sequence b: P keys already in the cache (post-prologue, chunked
// prefill only) and T new tokens; keys [0, P + T), query t is token P + t.
// A plain prefill has P = 0.
struct SeqExtent {
  int past, T, n;
};

__device__ __forceinline__ SeqExtent seq_extent(const PrefillParams& p, int b) {
  int P = p.past_lens ? p.past_lens[b] : 0;
  P = P < 0 ? 0 : (P > p.max_seq ? p.max_seq : P);
  const int tcap = min(p.max_chunk, p.max_seq - P);
  int T = p.seq_lens[b];
  T = T < 0 ? 0 : (T > tcap ? tcap : T);
  return SeqExtent{P, T, P + T};
}

// ----------------------------------------------------------------- phase 1: key prologue

// Eight bf16 (packed) to eight fp16 (packed), round to nearest even,
// saturating at +-65504.
__device__ __forceinline__ u32x4 bf16x8_to_f16x8(const u32x4 x) {
  return u32x4{pack_f16x2_sat(bf16lo(x[0]), bf16hi(x[0])), pack_f16x2_sat(bf16lo(x[1]), bf16hi(x[1])),
               pack_f16x2_sat(bf16lo(x[2]), bf16hi(x[2])), pack_f16x2_sat(bf16lo(x[3]), bf16hi(x[3]))};
}

// 16 key rows per workgroup; a row is held by 16 lanes (dims 4c..4c+3 and
// 64+4c..64+4c+3), so RMSNorm reduces over 16 lanes and RoPE pairs (i, i+64)
// stay in one lane.  The same lanes copy the row's V (16 bytes each).  Rows
// below P (chunked prefill) are already post-prologue and are copied as is.
__global__ __launch_bounds__(256) void key_prologue_kernel(const PrefillParams p, uint8_t* kws, uint8_t* vws) {
  __shared__ double inv_rev[kHeadDim / 2];
  const int b = blockIdx.z, h = blockIdx.y;
  const int tid = threadIdx.x, r = tid >> 4, c = tid & 15;
  // the attention kernel's arrival counters are zeroed here on every call (the
  // workspace's contents on entry are ignored); the attention kernel leaves
  // them at zero again
  if (p.counters != nullptr && b == 0 && h == 0)
    for (int i = blockIdx.x * 256 + tid; i < p.n_counters; i += gridDim.x * 256) p.counters[i] = 0;
  const bool rope = p.rope_theta > 0.0;
  if (tid < 64 && rope) inv_rev[tid] = rope_inv_freq(tid, p.rope_log2_theta) * 0.15915494309189535;
  __syncthreads();
  const SeqExtent ext = seq_extent(p, b);
  const int n = ext.n;
  const int key = blockIdx.x * 16 + r;
  const int64_t tile = ((int64_t)b * p.num_kv_heads + h) * ws_tiles(p.max_seq) + key / kBN;
  uint8_t* kd = kws + tile * kTileBytes + (key % kBN) * kKPitch;
  uint8_t* vd = vws + tile * kTileBytes + (key % kBN) * kVPitch;
  if (key >= n) {   // whole 16-lane groups take this branch together
    if (key < (n + kBN - 1) / kBN * kBN) {   // rows of the last, partial tile: zeros
      *(u32x4*)(kd + 16 * c) = u32x4{0, 0, 0, 0};
      *(u32x4*)(vd + 16 * c) = u32x4{0, 0, 0, 0};
    }
    return;
  }
  int64_t kro, vro;   // element offsets of cache row `key`: contiguous, or page / row through the block table
  if (p.block_table) {
    const int64_t page = p.block_table[(int64_t)b * p.max_blocks + (key >> p.block_log2)];
    const int64_t row = key & ((1 << p.block_log2) - 1);
    kro = page * p.k_sb + (int64_t)h * p.k_sh + row * p.k_ss;
    vro = page * p.v_sb + (int64_t)h * p.v_sh + row * p.v_ss;
  } else {
    kro = (int64_t)b * p.k_sb + (int64_t)h * p.k_sh + (int64_t)key * p.k_ss;
    vro = (int64_t)b * p.v_sb + (int64_t)h * p.v_sh + (int64_t)key * p.v_ss;
  }
  *(u32x4*)(vd + 16 * c) = bf16x8_to_f16x8(*(const u32x4*)((const uint8_t*)p.v + vro * 2 + 16 * c));
  const uint16_t* src = (const uint16_t*)p.k + kro;
  if (key < ext.past) {   // cached key: already transformed
    *(u32x4*)(kd + 16 * c) = bf16x8_to_f16x8(*(const u32x4*)((const uint8_t*)src + 16 * c));
    return;
  }
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
  *(u32x2*)(kd + 8 * c) = u32x2{pack_f16x2_sat(x[0], x[1]), pack_f16x2_sat(x[2], x[3])};
  *(u32x2*)(kd + 128 + 8 * c) = u32x2{pack_f16x2_sat(x[4], x[5]), pack_f16x2_sat(x[6], x[7])};
  // the cache keeps post-prologue keys: the row these 16 lanes (and nothing
  // else in this call) have just read receives k' rounded to bf16
  if (p.write_k_cache && (p.k_norm_w || rope)) {
    uint16_t* dst = (uint16_t*)p.k + kro;
    *(u32x2*)(dst + 4 * c) = u32x2{pack_bf16x2(x[0], x[1]), pack_bf16x2(x[2], x[3])};
    *(u32x2*)(dst + 64 + 4 * c) = u32x2{pack_bf16x2(x[4], x[5]), pack_bf16x2(x[6], x[7])};
  }
}

// ----------------------------------------------------------------- phase 2: attention

#define LDS_AS __attribute__((address_space(3)))

// One 1 KiB direct-to-LDS copy: lane l's 16 bytes at src + lane_off (lane_off
// = 16 l) land at LDS bytes lds + 16 l.  Issued from inline assembly so that
// the compiler does not wait for it before unrelated LDS reads; completion is
// waited for explicitly (s_waitcnt vmcnt) before the barrier that publishes
// the tile.  M0 carries the LDS address; nothing else in these kernels uses M0.
__device__ __forceinline__ void dma16(uint32_t lds, const uint8_t* src, uint32_t lane_off) {
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
  asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, %2" ::"s"(lds), "v"(lane_off), "s"(src)
               : "memory", "m0");
#pragma clang diagnostic pop
}

// A tile is NLD KiB contiguous in the workspace and in LDS; wave w issues
// copies w, w + 2, ...
template <int NLD>
__device__ __forceinline__ void dma_tile(uint32_t lds, const uint8_t* src, uint32_t lane_off, int wave) {
#pragma unroll
  for (int i = 0; i < (NLD + kWaves - 1) / kWaves; ++i) {
    const int c = kWaves * i + wave;
    if (c < NLD) dma16(lds + 1024u * c, src + 1024 * c, lane_off);
  }
}

// Query operand slots: lane (n32, hf) holds, for slot kk, dims 32hf + 8kk ..
// +7 (kk < 4) and 64 + 32hf + 8(kk-4) .. +7 (kk >= 4), so every query RoPE
// pair (i, i+64) stays in one lane; the K' operand of slot kk is read from the
// same dims of the lane's key row.

// S^T for the 32 keys of a K' tile and the wave's 32-row blocks:
// s[rb][i] = init[rb] + S[key 8(i/4) + 4hf + i%4][query 32rb + n32].  The
// query fragments carry the softmax scale times log2(e), so S is already in
// log2 units, and init = -m (the row's running maximum) leaves exp2(s) to the
// softmax: the subtraction rides in the accumulator's initial value.  Each K'
// fragment read from LDS feeds every block.  The seed is written with explicit
// 64-bit moves, nine instructions where the compiler emits sixteen 32-bit
// ones; per tile that made the attention kernel 2 % faster.  ZERO (the first
// tile) leaves the zero initial value to the products.
typedef __attribute__((ext_vector_type(8))) uint64_t u64x8;

template <bool ZERO>
__device__ __forceinline__ void qk_tile(f32x16 (&s)[kRB], const LDS_AS uint8_t* kt, const f16x8 (&qf)[kRB][8], int n32,
                                        int hf, const float (&init)[kRB]) {
  const LDS_AS uint8_t* base = kt + kKPitch * n32 + 64 * hf;
#pragma unroll
  for (int rb = 0; rb < kRB; ++rb) {
    if constexpr (ZERO) {
#pragma unroll
      for (int i = 0; i < 16; ++i) s[rb][i] = 0.f;
    } else {
      const uint64_t pair = ((uint64_t)__float_as_uint(init[rb]) << 32) | __float_as_uint(init[rb]);
      u64x8 seed;
#pragma unroll
      for (int i = 0; i < 7; ++i) {
        uint64_t x;
        // volatile: seven identical moves would otherwise be merged into one
        asm volatile("v_mov_b64 %0, %1" : "=v"(x) : "v"(pair));
        seed[i] = x;
      }
      seed[7] = pair;
      s[rb] = __builtin_bit_cast(f32x16, seed);
    }
  }
#pragma unroll
  for (int kk = 0; kk < 8; ++kk) {
    const u32x4 a = *(const LDS_AS u32x4*)(base + 16 * ((kk & 3) + 8 * (kk >> 2)));
#pragma unroll
    for (int rb = 0; rb < kRB; ++rb)
      s[rb] = __builtin_amdgcn_mfma_f32_32x32x16_f16(as_f16x8(a), qf[rb][kk], s[rb], 0, 0, 0);
  }
}

// IEEE maximum (NaN-propagating) needs no quieting of its MFMA-produced
// operands, and pairs of it fuse into v_maximum3: 8 instructions for the 16
// scores a lane holds of one row.
__device__ __forceinline__ float max3(float a, float b, float c) {
  return __builtin_elementwise_maximum(__builtin_elementwise_maximum(a, b), c);
}

__device__ __forceinline__ float row_max16(const f32x16& s) {
  float t[5];
#pragma unroll
  for (int i = 0; i < 5; ++i) t[i] = max3(s[3 * i], s[3 * i + 1], s[3 * i + 2]);
  return max3(max3(t[0], t[1], t[2]), t[3], __builtin_elementwise_maximum(t[4], s[15]));
}

// Online softmax in log2 units with a lazy rescale.  Keys at tile offsets at
// or past lim[rb] (per lane half) are invisible; row_max is the row maximum
// of each block (relative to m once the scores carry -m).
__device__ __forceinline__ void apply_mask(f32x16 (&s)[kRB], const int (&lim)[kRB]) {
#pragma unroll
  for (int rb = 0; rb < kRB; ++rb)
#pragma unroll
    for (int i = 0; i < 16; ++i) s[rb][i] = (8 * (i >> 2) + (i & 3) < lim[rb]) ? s[rb][i] : -INFINITY;
}

__device__ __forceinline__ void row_max(const f32x16 (&s)[kRB], float (&mx)[kRB]) {
#pragma unroll
  for (int rb = 0; rb < kRB; ++rb) {   // the two lane halves hold the row's two key halves
    float a, b;
    pair_xor32(row_max16(s[rb]), a, b);
    mx[rb] = __builtin_elementwise_maximum(a, b);
  }
}

// P = exp2(s) = exp2(S scale log2(e) - m) as fp16 MFMA operands pf[rb][e] (keys 16e +
// {4hf+t, 8+4hf+t}, t < 4).  The row sum l is taken over the fp16-rounded P
// that the P V products use (v_dot2 of each packed pair with (1, 1)), so
// numerator and denominator see the same weights.
__device__ __forceinline__ void softmax_exp(f32x16 (&s)[kRB], float (&l)[kRB], u32x4 (&pf)[kRB][2]) {
  const f16x2 one = {(_Float16)1.0f, (_Float16)1.0f};
#pragma unroll
  for (int rb = 0; rb < kRB; ++rb) {
#pragma unroll
    for (int i = 0; i < 16; ++i) s[rb][i] = fast_exp2(s[rb][i]);
#pragma unroll
    for (int e = 0; e < 2; ++e)
      pf[rb][e] = u32x4{pack_f16x2(s[rb][8 * e + 0], s[rb][8 * e + 1]), pack_f16x2(s[rb][8 * e + 2], s[rb][8 * e + 3]),
                        pack_f16x2(s[rb][8 * e + 4], s[rb][8 * e + 5]), pack_f16x2(s[rb][8 * e + 6], s[rb][8 * e + 7])};
    float ps[2] = {l[rb], 0.f};   // two chains, the first continuing the running sum
#pragma unroll
    for (int e = 0; e < 2; ++e)
#pragma unroll
      for (int w = 0; w < 4; ++w)   // the (uint32_t) copy matters: hipcc bit-casts element 0 of a vector lvalue
        ps[w & 1] = __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2, (uint32_t)pf[rb][e][w]), one, ps[w & 1],
                                           false);
    l[rb] = ps[0] + ps[1];
  }
}

// O^T += V^T P^T.  The V^T operand of MFMA e, dim tile T comes from two
// transposing reads of natural V rows: lane group g (16 lanes) covers dims
// 32T + 16(g%2) .. +15 and keys R = 16e + 8a + 4(g/2) .. R+3 for a = 0, 1
// (slots 4a .. 4a+3); source lane j of the group points at key R + j/4,
// dims + 4(j%4) .. +3.  Each V^T fragment feeds both row blocks.  The
// transposing read moves 16-bit elements as they are: the words are fp16,
// the builtin's bf16 vector type only fixes their width.
typedef __attribute__((__vector_size__(4 * sizeof(__bf16)))) __bf16 bf16x4_v;

__device__ __forceinline__ void pv_tile(f32x16 (&o)[kRB][4], const LDS_AS uint8_t* vt, const u32x4 (&pf)[kRB][2],
                                        int lane) {
  const int g = lane >> 4, j = lane & 15;
  const LDS_AS uint8_t* base = vt + kVPitch * (4 * (g >> 1) + (j >> 2)) + 2 * (16 * (g & 1) + 4 * (j & 3));
#pragma unroll
  for (int e = 0; e < 2; ++e)
#pragma unroll
    for (int T = 0; T < 4; ++T) {
      const bf16x4_v x0 =
          __builtin_amdgcn_ds_read_tr16_b64_v4bf16((LDS_AS bf16x4_v*)(base + kVPitch * (16 * e) + 64 * T));
      const bf16x4_v x1 =
          __builtin_amdgcn_ds_read_tr16_b64_v4bf16((LDS_AS bf16x4_v*)(base + kVPitch * (16 * e + 8) + 64 * T));
      const f16x8 a = __builtin_bit_cast(f16x8, __builtin_shufflevector(x0, x1, 0, 1, 2, 3, 4, 5, 6, 7));
#pragma unroll
      for (int rb = 0; rb < kRB; ++rb)
        o[rb][T] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, as_f16x8(pf[rb][e]), o[rb][T], 0, 0, 0);
    }
}

struct WaveState {
  f32x16 o[kRB][4];   // O^T: o[rb][T][4a + r] = O[query 32rb + n32][dim 32T + 8a + 4hf + r]
  float m[kRB], l[kRB];
};

// ---- split key ranges ("ADR-0060: AHBM GQA Fused Attention Kernel
// (Llama3-70B)" section 4: partials (m, l, O) of disjoint key ranges combine
// by the log-sum-exp merge).  When the grid is short (few query blocks), a
// query block whose visible keys span more than span_tiles tiles is cut
// into ns = ceil(tiles / span_tiles) nearly equal key spans, one workgroup
// each, so that more of the GPU works on it.  Each span writes its
// unnormalised state in the lanes' own register layout, then arrives at the
// block's counter; the last to arrive reads every span's state back (its own
// too: the tile loop's registers are dead by then), merges and writes out.
// Partial stores and loads are device-coherent (they bypass the
// non-coherent per-XCD L2s); a workgroup's stores have completed before its
// arrival.  No workgroup waits for another.
static_assert(kRB == 1, "partial layout: one 32-row block per wave");
constexpr int kPartO = kWaves * 16 * 64 * 4;           // floats of O: [wave][j][lane][4]
constexpr int kPartFloats = kPartO + kWaves * 64 * 2;  // + (m, l) per lane
constexpr int kMaxOrder = 1024;

// Workgroup order of the (query block, span) items of one (sequence, head):
// rank -> qb * n_spans + span, largest estimated item first; n == 0 means
// query blocks in descending order, spans in order.
struct AttnOrder {
  uint16_t item[kMaxOrder];
  int32_t n;
};

// Device-scope (sc1) buffer accesses to one partial slot: written through to,
// and read from, the device coherence point, past the per-XCD L2s.  The
// resource spans the slot only (accesses beyond it would be dropped).
constexpr int kDeviceScope = 16;   // cache-policy bit sc1
__device__ __forceinline__ __amdgpu_buffer_rsrc_t slot_rsrc(const float* slot) {
  return __builtin_amdgcn_make_buffer_rsrc((void*)slot, 0, kPartFloats * 4, 0x00020000);
}

__device__ __forceinline__ void store_partial(const float* slot, const WaveState& ws, int wave, int lane) {
  const __amdgpu_buffer_rsrc_t r = slot_rsrc(slot);
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    const f32x4 v = {ws.o[0][j >> 2][4 * (j & 3)], ws.o[0][j >> 2][4 * (j & 3) + 1], ws.o[0][j >> 2][4 * (j & 3) + 2],
                     ws.o[0][j >> 2][4 * (j & 3) + 3]};
    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, v), r, ((wave * 16 + j) * 64 + lane) * 16, 0,
                                           kDeviceScope);
  }
  __builtin_amdgcn_raw_buffer_store_b64(u32x2{__float_as_uint(ws.m[0]), __float_as_uint(ws.l[0])}, r,
                                        (kPartO + (wave * 64 + lane) * 2) * 4, 0, kDeviceScope);
}

__device__ __forceinline__ f32x4 load_o4(__amdgpu_buffer_rsrc_t r, int wave, int j, int lane) {
  return __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(r, ((wave * 16 + j) * 64 + lane) * 16, 0,
                                                                          kDeviceScope));
}

__device__ __forceinline__ void load_ml(__amdgpu_buffer_rsrc_t r, int wave, int lane, float& m, float& l) {
  const u32x2 v = __builtin_amdgcn_raw_buffer_load_b64(r, (kPartO + (wave * 64 + lane) * 2) * 4, 0, kDeviceScope);
  m = __uint_as_float(v[0]);
  l = __uint_as_float(v[1]);
}

__device__ __forceinline__ void load_partial(WaveState& ws, const float* slot, int wave, int lane) {
  const __amdgpu_buffer_rsrc_t r = slot_rsrc(slot);
  load_ml(r, wave, lane, ws.m[0], ws.l[0]);
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    const f32x4 x = load_o4(r, wave, j, lane);
#pragma unroll
    for (int i = 0; i < 4; ++i) ws.o[0][j >> 2][4 * (j & 3) + i] = x[i];
  }
}

// ws <- merge(ws, the partial in slot): M = max(m, m'), scale each side by 2^(m - M).
__device__ __forceinline__ void merge_partial(WaveState& ws, const float* slot, int wave, int lane) {
  const __amdgpu_buffer_rsrc_t r = slot_rsrc(slot);
  float mk, lk;
  load_ml(r, wave, lane, mk, lk);
  const float M = __builtin_elementwise_maximum(ws.m[0], mk);   // both finite: every row sees each span
  const float a = fast_exp2(ws.m[0] - M), c = fast_exp2(mk - M);
  ws.l[0] = a * ws.l[0] + c * lk;
  ws.m[0] = M;
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    const f32x4 x = load_o4(r, wave, j, lane);
#pragma unroll
    for (int i = 0; i < 4; ++i) ws.o[0][j >> 2][4 * (j & 3) + i] = a * ws.o[0][j >> 2][4 * (j & 3) + i] + c * x[i];
  }
}

struct WaveCtx {
  int wq0;          // first query row of the wave (of the T new tokens)
  int qrow[kRB];    // this lane's query row in each block
  int past;         // keys before the first query (query t is key P + t)
  int n;            // keys: P + T
  int wtiles;       // tiles holding keys this wave sees
  bool causal;
  // tile offsets at or past lim are invisible to this lane (per block)
  __device__ __forceinline__ void limits(int ks, int hf, int (&lim)[kRB]) const {
#pragma unroll
    for (int rb = 0; rb < kRB; ++rb) lim[rb] = (causal ? min(n, past + qrow[rb] + 1) : n) - ks - 4 * hf;
  }
  __device__ __forceinline__ bool needs_mask(int ks) const {   // wave-uniform
    return (causal && ks + kBN - 1 > past + wq0) || ks + kBN > n;
  }
};

// Tile t of the wave (t < wtiles): the scores of tile t+1 (K'_{t+1} in
// kt_next) go to s_next beside the exponentials of s_cur (tile t), then P V of
// tile t (V_t in vt) beside the row maxima of tile t+1 (taken before the
// diagonal tiles' masking branch, so that they share the products' basic
// block, and taken again after it on those tiles).  On the wave's last
// tile the scores and maxima are computed from whatever kt_next holds and
// discarded, which keeps the loop body one basic block apart from the masking
// of the diagonal tiles and the (rare) rescale.  The scores of tile t+1 are
// formed relative to the m of tile t; m grows to the new maxima when any of
// them exceeds m by more than 2^8 (wave-uniform decision); O and l follow,
// after the P V products that used the old m, and the fresh scores drop the
// increase.
__device__ __forceinline__ void wave_tile(int t, f32x16 (&s_cur)[kRB], f32x16 (&s_next)[kRB],
                                          const LDS_AS uint8_t* kt_next, const LDS_AS uint8_t* vt,
                                          const f16x8 (&qf)[kRB][8], WaveState& ws, const WaveCtx& w, int lane) {
  const int n32 = lane & 31, hf = lane >> 5;
  u32x4 pf[kRB][2];
  float neg_m[kRB];
#pragma unroll
  for (int rb = 0; rb < kRB; ++rb) neg_m[rb] = -ws.m[rb];
  qk_tile<false>(s_next, kt_next, qf, n32, hf, neg_m);
  softmax_exp(s_cur, ws.l, pf);
  float mx[kRB];   // row maxima of tile t+1 less m, in the block of the products
  row_max(s_next, mx);
  pv_tile(ws.o, vt, pf, lane);
  const int ks = (t + 1) * kBN;
  if (w.needs_mask(ks)) {   // a diagonal tile: its maxima again, after the mask
    int lim[kRB];
    w.limits(ks, hf, lim);
    apply_mask(s_next, lim);
    row_max(s_next, mx);
  }
  bool grow = false;
#pragma unroll
  for (int rb = 0; rb < kRB; ++rb) grow = grow || mx[rb] > kLazyRescale;
  if (t + 1 < w.wtiles && __any(grow)) {
#pragma unroll
    for (int rb = 0; rb < kRB; ++rb) {
      const float inc = __builtin_elementwise_maximum(mx[rb], 0.0f);
      const float corr = fast_exp2(-inc);
      ws.l[rb] *= corr;
#pragma unroll
      for (int T = 0; T < 4; ++T) ws.o[rb][T] *= corr;
      ws.m[rb] += inc;
#pragma unroll
      for (int i = 0; i < 16; ++i) s_next[rb][i] -= inc;
    }
  }
}

// out rows of this lane: O / l (l summed over the two lane halves).
__device__ __forceinline__ void write_rows(const PrefillParams& p, const WaveState& ws, const WaveCtx& wc, int b, int hq,
                                           int T, int hf) {
#pragma unroll
  for (int rb = 0; rb < kRB; ++rb) {
    const float l = sum_xor32(ws.l[rb]);
    if (wc.qrow[rb] >= T) continue;
    const float inv = 1.0f / l;
    uint8_t* orow = (uint8_t*)p.out +
                    ((int64_t)b * p.o_sb + (int64_t)hq * p.o_sh + (int64_t)wc.qrow[rb] * p.o_ss) * (p.out_bf16 ? 2 : 4);
#pragma unroll
    for (int t = 0; t < 4; ++t) {
#pragma unroll
      for (int a = 0; a < 4; ++a) {
        const int d0 = 32 * t + 8 * a + 4 * hf;
        const float v0 = ws.o[rb][t][4 * a] * inv, v1 = ws.o[rb][t][4 * a + 1] * inv;
        const float v2 = ws.o[rb][t][4 * a + 2] * inv, v3 = ws.o[rb][t][4 * a + 3] * inv;
        if (p.out_bf16) *(u32x2*)(orow + 2 * d0) = u32x2{pack_bf16x2(v0, v1), pack_bf16x2(v2, v3)};
        else *(f32x4*)(orow + 4 * d0) = f32x4{v0, v1, v2, v3};
      }
    }
  }
}

// Pipeline per tile t (one barrier): at the start of step t the copies of
// K'_{t+2} (into the buffer of K'_t, whose scores were computed in step t-1)
// and of V_{t+1} (into the buffer of V_{t-1}) are issued; step t computes the
// scores of tile t+1 and the softmax and P V of tile t; the copies are waited
// for before the closing barrier.
__global__ __launch_bounds__(kAttnThreads, kWavesPerSimd) void attention_kernel(const PrefillParams p, const uint8_t* kws,
                                                                     const uint8_t* vws, const AttnOrder ord) {
  __shared__ __attribute__((aligned(16))) uint8_t kt0[kTileBytes], kt1[kTileBytes];
  __shared__ __attribute__((aligned(16))) uint8_t vt0[kTileBytes], vt1[kTileBytes];
  __shared__ double inv_rev[kHeadDim / 2];   // query RoPE: theta^(-2i/128) / (2 pi)
  __shared__ __attribute__((aligned(16))) float gam[kHeadDim];   // query norm weights
  __shared__ int last_span;                   // this workgroup merges its query block's spans
#ifdef GQA_TIMELINE
  __shared__ uint64_t tla[GQA_TIMELINE_SLOTS];
#endif
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
  GQA_STAMP(0);   // entry

  // ---- workgroup -> (sequence, KV head group, query head, 128-query block, key span)
  const int nqb = p.n_qblocks;
  const int per_group = nqb * p.n_spans * G;
  const int groups = p.batch * p.num_kv_heads;
  const int bid = blockIdx.x;
  int grp, wi;
  if (groups % kXcds == 0) {   // XCD-aware: a (sequence, KV head) group's workgroups share one XCD
    const int slot = bid / kXcds;
    grp = bid % kXcds + kXcds * (slot / per_group);
    wi = slot % per_group;
  } else {
    grp = bid / per_group;
    wi = bid % per_group;
  }
  const int b = grp / p.num_kv_heads, h = grp % p.num_kv_heads;
  const int rank = wi / G;   // largest item first
  const int hq = h * G + wi % G;
  int qb, span;
  if (ord.n > 0) {
    const int it = ord.item[rank];
    qb = it / p.n_spans;
    span = it % p.n_spans;
  } else {
    qb = nqb - 1 - rank / p.n_spans;
    span = rank % p.n_spans;
  }

  const SeqExtent ext = seq_extent(p, b);
  const int n = ext.n, T = ext.T;
  const int q0 = qb * kBM;
  if (q0 >= T) return;
  const int qe = min(q0 + kBM, T);
  const int kend = p.causal ? ext.past + qe : n;
  const int ntb = (kend + kBN - 1) / kBN;                            // tiles of the query block
  const int ns = p.n_spans > 1 ? (ntb + p.span_tiles - 1) / p.span_tiles : 1;   // its spans
  if (span >= ns) return;
  const int ta = (int)((int64_t)span * ntb / ns), tb = (int)((int64_t)(span + 1) * ntb / ns);   // tiles [ta, tb)
  const bool rope = p.rope_theta > 0.0;
  const double pos0 = (double)p.positions[b];

  WaveCtx wc;
  wc.wq0 = q0 + 32 * kRB * wave;
#pragma unroll
  for (int rb = 0; rb < kRB; ++rb) wc.qrow[rb] = wc.wq0 + 32 * rb + n32;
  wc.past = ext.past;
  wc.n = n;
  wc.causal = p.causal != 0;
  const bool wave_live = wc.wq0 < T;
  const int wkend = !wave_live ? 0 : (wc.causal ? min(n, ext.past + wc.wq0 + 32 * kRB) : n);
  wc.wtiles = min((wkend + kBN - 1) / kBN, tb);   // end of this wave's tiles in the span

  const int64_t slab = ((int64_t)b * p.num_kv_heads + h) * ws_tiles(p.max_seq) * kTileBytes;
  const uint8_t* kslab = kws + slab;
  const uint8_t* vslab = vws + slab;
  const uint32_t lane_off = 16u * lane;

  // ---- the q rows and the norm weights are requested first; the first tiles'
  //      copies go out once they have landed, and land during the query
  //      prologue (loads return in issue order: copies issued first would hold
  //      the q rows back)
  if (tid < 64 && rope) inv_rev[tid] = rope_inv_freq(tid, p.rope_log2_theta) * 0.15915494309189535;
  u32x4 gv = {0u, 0u, 0u, 0u};
  if (tid < 16 && p.q_norm_w) gv = *(const u32x4*)((const uint16_t*)p.q_norm_w + 8 * tid);

  // ---- query prologue: lane (n32, hf) owns rows wq0 + n32 and wq0 + 32 + n32
  //      of head hq, dims [32hf, 32hf+32) and [64+32hf, 64+32hf+32)
  f16x8 qf[kRB][8];
  {
    u32x4 qlo[kRB][4], qhi[kRB][4];
#pragma unroll
    for (int rb = 0; rb < kRB; ++rb) {
      if (wc.qrow[rb] < T) {
        const uint16_t* row =
            (const uint16_t*)p.q + ((int64_t)b * p.q_sb + (int64_t)hq * p.q_sh + (int64_t)wc.qrow[rb] * p.q_ss);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          qlo[rb][j] = *(const u32x4*)(row + 32 * hf + 8 * j);
          qhi[rb][j] = *(const u32x4*)(row + 64 + 32 * hf + 8 * j);
        }
      } else {
#pragma unroll
        for (int j = 0; j < 4; ++j) qlo[rb][j] = qhi[rb][j] = u32x4{0, 0, 0, 0};
      }
    }
    __builtin_amdgcn_s_waitcnt(0);   // this thread's q rows and table entries have landed
    GQA_STAMP(1);                    // q rows landed
    if (tid < 16 && p.q_norm_w) {
      *(f32x4*)&gam[8 * tid] = f32x4{bf16lo(gv[0]), bf16hi(gv[0]), bf16lo(gv[1]), bf16hi(gv[1])};
      *(f32x4*)&gam[8 * tid + 4] = f32x4{bf16lo(gv[2]), bf16hi(gv[2]), bf16lo(gv[3]), bf16hi(gv[3])};
    }
    dma_tile<kTileBytes / 1024>(k0a, kslab + ta * kTileBytes, lane_off, wave);
    dma_tile<kTileBytes / 1024>(v0a, vslab + ta * kTileBytes, lane_off, wave);
    if (tb - ta > 1) dma_tile<kTileBytes / 1024>(k1a, kslab + (ta + 1) * kTileBytes, lane_off, wave);
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");   // this wave's table and norm-weight writes are done
    // the tables are visible to every wave; no wait for the tile copies here
    // (the wavefront-scope fences keep LDS accesses on their side of the
    // barrier without waiting for outstanding loads)
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    const uint16_t* g = (const uint16_t*)p.q_norm_w;
#pragma unroll
    for (int rb = 0; rb < kRB; ++rb) {
      float r = 1.0f;
      if (g) {
        float ss = 0.f;
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const float a = bf16_elem(qlo[rb][j], e), c = bf16_elem(qhi[rb][j], e);
            ss += a * a + c * c;
          }
        ss = sum_xor32(ss);
        r = rsqrtf(ss * (1.0f / kHeadDim) + p.eps);
      }
      r *= p.scale_log2;   // q' carries the softmax scale times log2(e) (RoPE is linear)
      const double qpos = pos0 + (double)(ext.past + wc.qrow[rb]);
      float amax = 0.f;   // the largest |q'| of the lane (NaN if any is NaN)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        float xl[8], xh[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          xl[e] = bf16_elem(qlo[rb][j], e);
          xh[e] = bf16_elem(qhi[rb][j], e);
        }
        if (g) {
          const f32x4 gl0 = *(const f32x4*)&gam[32 * hf + 8 * j], gl1 = *(const f32x4*)&gam[32 * hf + 8 * j + 4];
          const f32x4 gh0 = *(const f32x4*)&gam[64 + 32 * hf + 8 * j], gh1 = *(const f32x4*)&gam[64 + 32 * hf + 8 * j + 4];
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            xl[e] *= r * (e < 4 ? gl0[e] : gl1[e - 4]);
            xh[e] *= r * (e < 4 ? gh0[e] : gh1[e - 4]);
          }
        } else {
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            xl[e] *= r;
            xh[e] *= r;
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
#pragma unroll
        for (int e = 0; e < 8; ++e)
          amax = __builtin_elementwise_maximum(__builtin_elementwise_maximum(amax, fabsf(xl[e])), fabsf(xh[e]));
        qf[rb][j] = as_f16x8(u32x4{pack_f16x2(xl[0], xl[1]), pack_f16x2(xl[2], xl[3]), pack_f16x2(xl[4], xl[5]),
                                   pack_f16x2(xl[6], xl[7])});
        qf[rb][4 + j] = as_f16x8(u32x4{pack_f16x2(xh[0], xh[1]), pack_f16x2(xh[2], xh[3]), pack_f16x2(xh[4], xh[5]),
                                       pack_f16x2(xh[6], xh[7])});
      }
      // fp16 saturation after the conversion, on the rare waves with an
      // element beyond 65504 (or a NaN, which the fix leaves as it is)
      if (__any(!(amax <= kF16Max))) {
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          u32x4 w = __builtin_bit_cast(u32x4, qf[rb][j]);
#pragma unroll
          for (int i = 0; i < 4; ++i) w[i] = saturate_inf_f16x2(w[i]);
          qf[rb][j] = as_f16x8(w);
        }
      }
    }
  }

  GQA_STAMP(2);   // query prologue done
  WaveState ws;
#pragma unroll
  for (int rb = 0; rb < kRB; ++rb) {
#pragma unroll
    for (int T = 0; T < 4; ++T)
#pragma unroll
      for (int i = 0; i < 16; ++i) ws.o[rb][T][i] = 0.f;
    ws.l[rb] = 0.f;
  }

  f32x16 sa[kRB], sb[kRB];
  __builtin_amdgcn_s_waitcnt(0);   // this thread's tile copies have landed
  __syncthreads();                 // K'_0, K'_1, V_0
  GQA_STAMP(3);                    // first tiles landed
  if (wc.wtiles > ta) {   // scores and row maxima of tile ta (every row sees the span's first key: m is finite)
    const float zero[kRB] = {};
    qk_tile<true>(sa, K0, qf, n32, hf, zero);
    if (wc.needs_mask(ta * kBN)) {
      int lim[kRB];
      wc.limits(ta * kBN, hf, lim);
      apply_mask(sa, lim);
    }
    row_max(sa, ws.m);
#pragma unroll
    for (int rb = 0; rb < kRB; ++rb)
#pragma unroll
      for (int i = 0; i < 16; ++i) sa[rb][i] -= ws.m[rb];
  }
  __syncthreads();   // every read of K'_ta done: its buffer takes K'_ta+2

  // two tiles per trip: buffers and score registers have fixed roles in each half
  for (int t = ta; t < tb; t += 2) {
    if (t + 2 < tb) dma_tile<kTileBytes / 1024>(k0a, kslab + (t + 2) * kTileBytes, lane_off, wave);
    if (t + 1 < tb) dma_tile<kTileBytes / 1024>(v1a, vslab + (t + 1) * kTileBytes, lane_off, wave);
    if (t < wc.wtiles) wave_tile(t, sa, sb, K1, V0, qf, ws, wc, lane);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    const int t1 = t + 1;
    if (t1 >= tb) break;
    if (t1 + 2 < tb) dma_tile<kTileBytes / 1024>(k1a, kslab + (t1 + 2) * kTileBytes, lane_off, wave);
    if (t1 + 1 < tb) dma_tile<kTileBytes / 1024>(v0a, vslab + (t1 + 1) * kTileBytes, lane_off, wave);
    if (t1 < wc.wtiles) wave_tile(t1, sb, sa, K0, V1, qf, ws, wc, lane);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
  }
#ifdef GQA_TIMELINE
  GQA_STAMP(4);   // tile loop done
  if (tid == 0) tla[6] = (uint64_t)(tb - ta);   // tiles of this workgroup
  __syncthreads();
  if (tid < GQA_TIMELINE_SLOTS && tid != 5 && blockIdx.x < GQA_TIMELINE_BLOCKS)
    g_timeline_attn[blockIdx.x * GQA_TIMELINE_SLOTS + tid] = tid == 7 ? 0 : tla[tid];
#endif
  // ---- a split block: store this span's state, arrive; the last span merges
  if (ns > 1) {
    const int64_t blk = ((int64_t)b * p.num_q_heads + hq) * nqb + qb;
    const float* part = p.partials + blk * p.n_spans * kPartFloats;
    if (wave_live) store_partial(p.partials + (blk * p.n_spans + span) * kPartFloats, ws, wave, lane);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");   // this thread's partial stores have completed
    __syncthreads();
    if (tid == 0) {
      const uint32_t prev = __hip_atomic_fetch_add(p.counters + blk, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      last_span = prev + 1 == (uint32_t)ns;
      // every span of the block has arrived: the counter is back to zero for
      // the next call, so the attention phase can be replayed on its own
      if (last_span) __hip_atomic_store(p.counters + blk, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    __syncthreads();
    if (!last_span) {
      GQA_STAMP_END();
      return;
    }
    if (!wave_live) return;
    // every span's state (this one's too) from memory: the tile loop's registers are dead here
    WaveState mg;
    load_partial(mg, part, wave, lane);
    for (int k = 1; k < ns; ++k) merge_partial(mg, part + k * kPartFloats, wave, lane);
    write_rows(p, mg, wc, b, hq, T, hf);
    GQA_STAMP_END();
    return;
  }
  // ---- epilogue: O / l for this lane's query rows
  if (!wave_live) return;
  write_rows(p, ws, wc, b, hq, T, hf);
  GQA_STAMP_END();   // wave 0 is live in every workgroup that gets here
}

// Split plan of the attention grid (host).  The work of a query block is
// estimated from the extent of the largest sequence the descriptor admits:
// T = max_chunk new tokens after max_seq - max_chunk cached ones.  Key spans
// are used only when the grid has fewer than 384 workgroups (1.5 per compute
// unit), where it cannot fill the GPU: a chunk after a long cached prefix,
// or one sequence with few heads.  Spans are then sized for about 640 items
// (2.5 workgroups per compute unit), at least 16 tiles and at most 16 per
// block.  Measured on Qwen3-14B shapes: a 1024-token chunk after 3072
// cached tokens takes 134 us unsplit, 119 us in 2 spans, 134 us in 3; a
// 96-token chunk after 4000, 104 us unsplit, 66 in 2 spans, 45 in 4, 41 in
// 8 (16 tiles per span; 8 tiles per span, 16 spans: 44 us, the last span's
// merge of 16 partials costing more than the shorter spans save); the
// 4096-token prefill (1280 workgroups) is not split, splitting its longest
// blocks made it 8 % slower.
struct SplitPlan {
  int n_qblocks, n_spans, span_tiles;
};

int est_block_tiles(int max_seq, int max_chunk, bool causal, int qb) {
  const int64_t past = (int64_t)max_seq - max_chunk;
  const int64_t qe = std::min<int64_t>((int64_t)(qb + 1) * kBM, max_chunk);
  const int64_t kend = causal ? past + qe : past + max_chunk;
  return (int)((kend + kBN - 1) / kBN);
}

SplitPlan split_plan(int batch, int num_q_heads, int max_seq, int max_chunk, bool causal) {
  SplitPlan sp{(max_chunk + kBM - 1) / kBM, 1, 0};
  const int tiles = (int)ws_tiles(max_seq);
  int longest = 0;
  for (int qb = 0; qb < sp.n_qblocks; ++qb) longest = std::max(longest, est_block_tiles(max_seq, max_chunk, causal, qb));
  const int64_t items = (int64_t)batch * num_q_heads * sp.n_qblocks;
  sp.span_tiles = (int)std::max<int64_t>({16, ((int64_t)longest * items + 639) / 640, (tiles + 15) / 16});
  if (items < 384 && longest > sp.span_tiles) sp.n_spans = (tiles + sp.span_tiles - 1) / sp.span_tiles;
  return sp;
}

// Items (query block, span) of one head sorted by estimated tiles, largest
// first (ties: later block first); n = 0 when they do not fit the table.
void fill_order(const SplitPlan& sp, int max_seq, int max_chunk, bool causal, AttnOrder& ord) {
  const int items = sp.n_qblocks * sp.n_spans;
  ord.n = 0;
  if (sp.n_spans == 1 || items > kMaxOrder) return;
  std::vector<std::pair<int, int>> key(items);   // (-estimated tiles, -item)
  for (int qb = 0; qb < sp.n_qblocks; ++qb) {
    const int t = est_block_tiles(max_seq, max_chunk, causal, qb);
    const int ns = (t + sp.span_tiles - 1) / sp.span_tiles;
    for (int sidx = 0; sidx < sp.n_spans; ++sidx) {
      const int size = sidx < ns ? (int)((int64_t)(sidx + 1) * t / ns - (int64_t)sidx * t / ns) : 0;
      key[qb * sp.n_spans + sidx] = {-size, -(qb * sp.n_spans + sidx)};
    }
  }
  std::sort(key.begin(), key.end());
  for (int r = 0; r < items; ++r) ord.item[r] = (uint16_t)(-key[r].second);
  ord.n = items;
}

// Workspace: [K' tiles][V tiles], then, for a split plan, [counters: B * Hq *
// n_qblocks u32, to 256 bytes][partials: B * Hq * n_qblocks * n_spans *
// kPartFloats f32].
size_t kv_bytes(int batch, int num_kv_heads, int max_seq) {
  return (size_t)batch * num_kv_heads * ws_tiles(max_seq) * kTileBytes * 2;
}

size_t split_bytes(int batch, int num_q_heads, const SplitPlan& sp) {
  if (sp.n_spans == 1) return 0;
  const size_t blocks = (size_t)batch * num_q_heads * sp.n_qblocks;
  return (blocks * 4 + 255) / 256 * 256 + blocks * sp.n_spans * kPartFloats * sizeof(float);
}

}  // namespace

size_t prefill_workspace_bytes(int batch, int num_q_heads, int num_kv_heads, int max_seq, int max_chunk, bool causal) {
  const size_t plain = split_bytes(batch, num_q_heads, split_plan(batch, num_q_heads, max_seq, max_seq, causal));
  const size_t chunk = split_bytes(batch, num_q_heads, split_plan(batch, num_q_heads, max_seq, max_chunk, causal));
  return kv_bytes(batch, num_kv_heads, max_seq) + std::max(plain, chunk);
}

hipError_t launch_prefill_phased(const PrefillParams& p, void* workspace, hipStream_t stream, int phases) {
  uint8_t* kws = (uint8_t*)workspace;
  uint8_t* vws = kws + (size_t)p.batch * p.num_kv_heads * ws_tiles(p.max_seq) * kTileBytes;
  const SplitPlan sp = split_plan(p.batch, p.num_q_heads, p.max_seq, p.max_chunk, p.causal != 0);
  PrefillParams q = p;
  q.n_qblocks = sp.n_qblocks;
  q.n_spans = sp.n_spans;
  q.span_tiles = sp.span_tiles;
  q.counters = nullptr;
  q.n_counters = 0;
  q.partials = nullptr;
  if (sp.n_spans > 1) {
    uint8_t* extra = kws + kv_bytes(p.batch, p.num_kv_heads, p.max_seq);
    const size_t blocks = (size_t)p.batch * p.num_q_heads * sp.n_qblocks;
    q.counters = (uint32_t*)extra;
    q.n_counters = (int32_t)blocks;
    q.partials = (float*)(extra + (blocks * 4 + 255) / 256 * 256);
  }
  AttnOrder ord;
  fill_order(sp, p.max_seq, p.max_chunk, p.causal != 0, ord);
  if (phases & kPhaseKeys) {
    const hipError_t e = launch_kernel(key_prologue_kernel,
                                       dim3((unsigned)(ws_tiles(p.max_seq) * kBN / 16), p.num_kv_heads, p.batch),
                                       dim3(256), stream, q, kws, vws);
    if (e != hipSuccess) return e;
  }
  if (!(phases & kPhaseAttend)) return hipSuccess;
  return launch_kernel(attention_kernel, dim3(q.n_qblocks * q.n_spans * p.num_q_heads * p.batch), dim3(kAttnThreads),
                       stream, q, (const uint8_t*)kws, (const uint8_t*)vws, ord);
}

#ifdef GQA_TIMELINE
hipError_t timeline_attn_clear(const uint64_t* zeros, size_t bytes) {
  return hipMemcpyToSymbol(HIP_SYMBOL(g_timeline_attn), zeros, bytes);
}
hipError_t timeline_attn_read(uint64_t* host, size_t bytes) {
  return hipMemcpyFromSymbol(host, HIP_SYMBOL(g_timeline_attn), bytes);
}
#endif

}  // namespace gqa
