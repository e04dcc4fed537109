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
//  * one workgroup = (chunk c, KV head h, sequence b) on a 1-D grid whose
//    chunks of one (b, h) share an XCD when the group count allows; in a
//    batch the chunks that hold keys come ahead of those past their
//    sequence's end (the lengths are read on the device), a single
//    sequence's map is static so that its q rows are requested while its
//    length is read; 4 streaming waves + 1 prologue wave.  Streaming wave w handles 32-key
//    steps w, w+4, ... of the chunk with its own online-softmax state; the 4
//    states are merged through LDS at the end.
//  * The prologue wave has its own in-order memory queue: it loads q, the
//    norm weights and the new key row while the streaming waves' K/V loads
//    are in flight, builds the RoPE table, writes q' (f32 and bf16 hi/lo) to
//    LDS, and computes the score of the new key (slot L-1) exactly in f32,
//    which replaces the matrix-core score of the raw cached row.
//  * S^T = K Q'^T and O^T = V^T P^T run on v_mfma_f32_16x16x32_bf16 (bf16
//    inputs; q' and P as bf16 hi + lo pairs) or v_mfma_f32_16x16x4_f32 (f32
//    inputs) with the G <= 16 query rows as the 16-wide N dimension; a lane
//    owns one query head (lane % 16), and the 8x8 bf16 transpose that V^T
//    needs is done in registers.
//  * Memory requests of one compute unit are served in issue order, so the
//    prologue wave issues its small loads (q, norm weights, the new key row)
//    before the streaming waves start the K/V stream, behind a workgroup
//    barrier.
#include "common.hpp"
#ifdef GQA_TIMELINE
#include "gqa_timeline.h"
#endif

namespace gqa {
namespace {

constexpr int kXcds = 8;
constexpr int kStreamWaves = 4;
constexpr int kPrologueWave = kStreamWaves;
constexpr int kThreads = (kStreamWaves + 1) * 64;
// Single-chunk grids of many workgroups run a 4-wave form instead: streaming
// wave 0 also runs the prologue and one chunk-state buffer suffices, so two
// workgroups share a compute unit (two waves per SIMD, no register spills) and
// one's start (lengths, q rows, prologue) overlaps the other's K/V stream.
constexpr int kThreads4 = kStreamWaves * 64;
constexpr int kMany4 = 1024;   // grids of at least this many single-chunk workgroups
constexpr int kStep = 32;        // keys per wave step
constexpr int kORow = 132;       // padded LDS row (floats) of the in-workgroup merge
constexpr int kQRow = 136;       // padded bf16 q' row (272 bytes): 16 rows x 16 bytes hit distinct banks

// Per-workgroup timeline of the partition kernel, compiled in only with
// -DGQA_TIMELINE (a separate measurement build of the library): one lane
// takes s_memrealtime stamps into LDS at fixed points (include/gqa_timeline.h
// lists them) and the workgroup writes them out once at its end, so the timed
// path gets no global memory instruction.  Without the flag the stamps
// expand to nothing (not even their conditions).
#ifdef GQA_TIMELINE
constexpr int kTimelineSlots = GQA_TIMELINE_SLOTS;
constexpr int kTimelineBlocks = GQA_TIMELINE_BLOCKS;
__device__ uint64_t g_timeline[kTimelineBlocks * kTimelineSlots];
#define GQA_STAMP(cond, i) \
  do {                        \
    if (cond) tl[(i)] = __builtin_amdgcn_s_memrealtime(); \
  } while (0)
#else
#define GQA_STAMP(cond, i)
#endif

template <int NB>   // chunk-state buffers: 2 when a workgroup sweeps several chunks
struct __attribute__((aligned(16))) DecodeSmemT {
  float cs[64][2];               // RoPE cos / sin at positions[b]
  float qp[16][kHeadDim];        // q' rows after the prologue (rows >= G are zero)
  uint16_t qh[16][kQRow];        // bf16(q')            (rows >= G are zero)
  uint16_t ql[16][kQRow];        // bf16(q' - bf16(q'))
  float kn[kHeadDim];            // the new key row after the prologue
  float snew[16];                // score of the new key per query head (log2 units)
  float mo[NB][kStreamWaves][16][kORow];   // per-wave unnormalised O of a chunk (double-buffered when NB = 2)
  float mm[NB][kStreamWaves][16];
  float ml[NB][kStreamWaves][16];
};

// Half-row fetch of a 128-element row for the 16 lanes that hold it:
// elements 4*c16 .. 4*c16+3 and 64+4*c16 .. 64+4*c16+3.  The raw words are
// kept until unpack_half_row, so that a fetch issued early is not waited on.
template <bool BF16> struct RawHalf;
template <> struct RawHalf<true> { u32x2 lo, hi; };
template <> struct RawHalf<false> { f32x4 lo, hi; };

template <bool BF16>
__device__ __forceinline__ RawHalf<BF16> fetch_half_row(const void* row, int c16) {
  RawHalf<BF16> r;
  if constexpr (BF16) {
    r.lo = *(const u32x2*)((const uint16_t*)row + 4 * c16);
    r.hi = *(const u32x2*)((const uint16_t*)row + 64 + 4 * c16);
  } else {
    r.lo = *(const f32x4*)((const float*)row + 4 * c16);
    r.hi = *(const f32x4*)((const float*)row + 64 + 4 * c16);
  }
  return r;
}

template <bool BF16>
__device__ __forceinline__ void unpack_half_row(const RawHalf<BF16>& r, float (&x)[8]) {
  if constexpr (BF16) {
    x[0] = bf16lo(r.lo[0]); x[1] = bf16hi(r.lo[0]); x[2] = bf16lo(r.lo[1]); x[3] = bf16hi(r.lo[1]);
    x[4] = bf16lo(r.hi[0]); x[5] = bf16hi(r.hi[0]); x[6] = bf16lo(r.hi[1]); x[7] = bf16hi(r.hi[1]);
  } else {
#pragma unroll
    for (int j = 0; j < 4; ++j) { x[j] = r.lo[j]; x[4 + j] = r.hi[j]; }
  }
}

// The prologue on one row held by 16 consecutive lanes (8 elements each):
// RMSNorm over the 128 elements (skipped if !norm), then RoPE with the cos /
// sin table (skipped if !rope).  All 16 lanes must be active.
__device__ __forceinline__ void prologue_row(float (&x)[8], int c16, bool norm, const float (&g)[8], float eps,
                                             bool rope, const float (*cs)[2]) {
  if (norm) {
    float ss = 0.f;
    #pragma unroll
    for (int j = 0; j < 8; ++j) ss += x[j] * x[j];
    ss = sum16(ss);
    const float r = rsqrtf(ss * (1.0f / kHeadDim) + eps);
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
  u32x4 k[2][4];   // K rows key0 + 16*gi + (lane%16), dims 32*kb + 8*(lane/16) .. +8
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
// K / V rows of one (sequence, KV head).  Contiguous: row j at kb + j * kss.
// Paged: logical row j at kb + block_table[j >> log2bs] * kpage + (j % bs) * kss;
// steps start at multiples of 32 keys and pages hold a power of two >= 32
// rows, so the 32 rows of a step always share one page.
template <bool PAGED>
struct Slab {
  static constexpr bool kPaged = PAGED;
  const uint8_t* kb;
  const uint8_t* vb;
  uint32_t kss, vss;     // row strides in bytes
  uint32_t klane, vlane; // per-lane byte offsets
  const int32_t* bt;     // paged: this sequence's row of the block table
  int log2bs;            // paged: log2(rows per page)
  int64_t kpage, vpage;  // paged: page strides in bytes

  // The page holding key (paged; 0 otherwise).  key is clamped below kend,
  // so the table entry read is one of the sequence's own blocks.  The sweep
  // requests it one step ahead of the loads that use it.
  __device__ __forceinline__ int page_of(int key, int kend) const {
    if constexpr (PAGED) return bt[min(key, kend - 1) >> log2bs];
    else return 0;
  }
  // base pointers of `page` (the one holding key0) and key0's row index in it
  __device__ __forceinline__ const uint8_t* kbase(int key0, int page, int& rel) const {
    if constexpr (PAGED) {
      rel = key0 & ((1 << log2bs) - 1);
      return kb + (int64_t)page * kpage;
    } else {
      rel = key0;
      return kb;
    }
  }
  __device__ __forceinline__ const uint8_t* vbase(int key0, int page, int& rel) const {
    if constexpr (PAGED) {
      rel = key0 & ((1 << log2bs) - 1);
      return vb + (int64_t)page * vpage;
    } else {
      rel = key0;
      return vb;
    }
  }
};

// Loads of one step (bf16).  V is read non-temporally (streamed once, not
// kept in the caches): a V load instruction reads 4 whole rows.  K load
// instruction kb reads bytes 64 kb .. 64 kb + 63 of 16 rows (lane (n16, q4):
// row n16, dims 32 kb + 8 q4 .. +7; the q fragment holds the same dims), so
// the two instructions that share a cache line are issued back to back; K is
// read non-temporally over a contiguous cache and with the default policy over
// a paged one, where that measured faster.  (The arithmetic is the same on
// both, so paged and contiguous results are bitwise equal.)
// FULL: every row of the step is below kend, no
// predication.  !FULL (the last step of a chunk): rows at or past kend are
// replaced by row kend-1 (always valid), so rows past the sequence are never
// read.  Their values stay as loaded: the scores of keys at or past kend are
// masked to -inf, which makes their P exactly 0, so nothing waits on these
// loads here and both forms leave the same loads in flight.
template <bool FULL, class SL>
__device__ __forceinline__ void load_k(StepBF16& st, const SL& sl, int key0, int kend, int n16, int q4, int page) {
  constexpr bool kNT = !SL::kPaged;
  int rel;
  const uint8_t* kb = sl.kbase(key0, page, rel);
#pragma unroll
  for (int gi = 0; gi < 2; ++gi) {
    const int key = key0 + 16 * gi + n16;
    const bool ok = FULL || key < kend;
    const uint32_t off = FULL ? (uint32_t)(rel + 16 * gi) * sl.kss + sl.klane
                              : (uint32_t)((ok ? key : kend - 1) - key0 + rel) * sl.kss + 16u * q4;
    const u32x4* src = (const u32x4*)(kb + off);
#pragma unroll
    for (int j = 0; j < 4; ++j) st.k[gi][j] = kNT ? __builtin_nontemporal_load(&src[4 * j]) : src[4 * j];
  }
}

template <bool FULL, class SL>
__device__ __forceinline__ void load_v(StepBF16& st, const SL& sl, int key0, int kend, int n16, int q4, int page) {
  int rel;
  const uint8_t* vb = sl.vbase(key0, page, rel);
#pragma unroll
  for (int t = 0; t < 8; ++t) {
    const int key = key0 + 4 * q4 + vkey_t(t);
    const bool ok = FULL || key < kend;
    const uint32_t off = FULL ? (uint32_t)(rel + vkey_t(t)) * sl.vss + sl.vlane
                              : (uint32_t)((ok ? key : kend - 1) - key0 + rel) * sl.vss + 16u * n16;
    st.v[t] = __builtin_nontemporal_load((const u32x4*)(vb + off));
  }
}

template <bool FULL, class SL>
__device__ __forceinline__ void load_k(StepF32& st, const SL& sl, int key0, int kend, int n16, int q4, int page) {
  int rel;
  const uint8_t* kb = sl.kbase(key0, page, rel);
#pragma unroll
  for (int gi = 0; gi < 2; ++gi) {
    const int key = key0 + 16 * gi + n16;
    const bool ok = FULL || key < kend;
    const uint32_t off = FULL ? (uint32_t)(rel + 16 * gi) * sl.kss + sl.klane
                              : (uint32_t)((ok ? key : kend - 1) - key0 + rel) * sl.kss + 128u * q4;
    const f32x4* src = (const f32x4*)(kb + off);
#pragma unroll
    for (int j = 0; j < 8; ++j) st.k[gi][j] = src[j];
  }
}

template <bool FULL, class SL>
__device__ __forceinline__ void load_v(StepF32& st, const SL& sl, int key0, int kend, int n16, int q4, int page) {
  int rel;
  const uint8_t* vb = sl.vbase(key0, page, rel);
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const int key = key0 + 16 * (e >> 2) + 4 * q4 + (e & 3);
    const bool ok = FULL || key < kend;
    const uint32_t off = FULL ? (uint32_t)(rel + 16 * (e >> 2) + (e & 3)) * sl.vss + sl.vlane
                              : (uint32_t)((ok ? key : kend - 1) - key0 + rel) * sl.vss + 32u * n16;
    const f32x4* src = (const f32x4*)(vb + off);
    st.v[e][0] = src[0];
    st.v[e][1] = src[1];
  }
}

template <class Step, class SL>
__device__ __forceinline__ void load_k_any(Step& st, const SL& sl, int key0, int kend, int n16, int q4, int page) {
  if (key0 + kStep <= kend) load_k<true>(st, sl, key0, kend, n16, q4, page);
  else load_k<false>(st, sl, key0, kend, n16, q4, page);
}

template <class Step, class SL>
__device__ __forceinline__ void load_v_any(Step& st, const SL& sl, int key0, int kend, int n16, int q4, int page) {
  if (key0 + kStep <= kend) load_v<true>(st, sl, key0, kend, n16, q4, page);
  else load_v<false>(st, sl, key0, kend, n16, q4, page);
}

template <class Step, class SL>
__device__ __forceinline__ void load_step(Step& st, const SL& sl, int key0, int kend, int n16, int q4, int page) {
  load_k_any(st, sl, key0, kend, n16, q4, page);
  load_v_any(st, sl, key0, kend, n16, q4, page);
}

// ----------------------------------------------------------------- query operand and running state

// bf16 path: q' = hi + lo with hi = bf16(q'), lo = bf16(q' - hi), so the score
// keeps ~16 significant bits of q' (two MFMAs per product; decode has the
// matrix-core headroom).
struct QFragBF16 { bf16x8 hi[4], lo[4]; };
struct QFragF32 { float q[32]; };

template <class SM>
__device__ __forceinline__ void load_qfrag(QFragBF16& qf, const SM& sm, int n16, int q4) {
#pragma unroll
  for (int kb = 0; kb < 4; ++kb) {   // the dims lane (n16, q4) holds of K for product kb
    qf.hi[kb] = *(const bf16x8*)&sm.qh[n16][32 * kb + 8 * q4];
    qf.lo[kb] = *(const bf16x8*)&sm.ql[n16][32 * kb + 8 * q4];
  }
}

template <class SM>
__device__ __forceinline__ void load_qfrag(QFragF32& qf, const SM& sm, int n16, int q4) {
#pragma unroll
  for (int j = 0; j < 32; j += 4) {
    const f32x4 x = *(const f32x4*)&sm.qp[n16][32 * q4 + j];
    qf.q[j] = x[0]; qf.q[j + 1] = x[1]; qf.q[j + 2] = x[2]; qf.q[j + 3] = x[3];
  }
}

struct RunState {
  f32x4 o[8];      // O^T tiles: lane holds O[g = lane%16][dim (4*(lane/16)+i)*8 + T] in o[T][i]
  float m;         // running max (log2 units), same in the 4 lanes of one query head
  float l;         // this lane's share of the running normaliser
};

// scores: s[4*gi + i] = S[key key0 + 16*gi + 4*q4 + i][g = lane%16] (log2 units).
// Four independent accumulation chains (key group x hi / lo part of q').
__device__ __forceinline__ void scores(const StepBF16& st, const QFragBF16& qf, float scale_log2, float (&s)[8]) {
  f32x4 ah[2], al[2];
#pragma unroll
  for (int gi = 0; gi < 2; ++gi) ah[gi] = al[gi] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int kb = 0; kb < 4; ++kb)
#pragma unroll
    for (int gi = 0; gi < 2; ++gi) {
      ah[gi] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(st.k[gi][kb]), qf.hi[kb], ah[gi], 0, 0, 0);
      al[gi] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(st.k[gi][kb]), qf.lo[kb], al[gi], 0, 0, 0);
    }
#pragma unroll
  for (int gi = 0; gi < 2; ++gi)
#pragma unroll
    for (int i = 0; i < 4; ++i) s[4 * gi + i] = (ah[gi][i] + al[gi][i]) * scale_log2;
}

__device__ __forceinline__ void scores(const StepF32& st, const QFragF32& qf, float scale_log2, float (&s)[8]) {
#pragma unroll
  for (int gi = 0; gi < 2; ++gi) {
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int j = 0; j < 8; ++j)
#pragma unroll
      for (int e = 0; e < 4; ++e)
        acc = __builtin_amdgcn_mfma_f32_16x16x4f32(st.k[gi][j][e], qf.q[4 * j + e], acc, 0, 0, 0);
#pragma unroll
    for (int i = 0; i < 4; ++i) s[4 * gi + i] = acc[i] * scale_log2;
  }
}

// O^T += V^T P^T.  bf16 path: P = hi + lo (two MFMAs per tile).
__device__ __forceinline__ void accumulate_pv(const StepBF16& st, const float (&p)[8], RunState& rs) {
  // P^T operand: slot t of lane group q4 <-> key vkey_t(t) of that group = the
  // score order p[0..7] of this lane.
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
// Refill (kRefill, or kRefillIfMore when next_key0 < kend): the step at
// next_key0 is requested into st, its K half right after the QK^T MFMAs have
// consumed st.k, its V half right after P V has consumed st.v.  (The bf16
// sweep gives a wave's last step no refill and leaves the step loop with it,
// so on the loop's back edge K and V are always in flight in that order and
// the compiler's wait counts let the QK^T products wait for K only.)
// kn >= 0: the score of key kn (the new key) is replaced by snew[lane % 16].
// page: the page of next_key0 (paged caches), requested a step earlier; on
// return it holds the page of the step after next_key0.
enum RefillMode { kNoRefill, kRefill, kRefillIfMore };

template <RefillMode REFILL, class Step, class QFrag, class SL>
__device__ __forceinline__ void sweep_step(Step& st, const QFrag& qf, const float* snew, int kn, RunState& rs,
                                           float scale_log2, int key0, int kend, int next_key0, const SL& sl,
                                           int n16, int q4, int& page) {
  const bool full = key0 + kStep <= kend;
  float s[8];
  scores(st, qf, scale_log2, s);
  const bool more = REFILL == kRefill || (REFILL == kRefillIfMore && next_key0 < kend);
  if (more) load_k_any(st, sl, next_key0, kend, n16, q4, page);
  if (kn >= key0 && kn < key0 + kStep) {   // wave-uniform: this step holds the new key
    const float sn = snew[n16];
#pragma unroll
    for (int e = 0; e < 8; ++e)
      if (key0 + 16 * (e >> 2) + 4 * q4 + (e & 3) == kn) s[e] = sn;
  }
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
  mx = max_xor32(max_xor16(mx));
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
  if (more) {
    load_v_any(st, sl, next_key0, kend, n16, q4, page);
    page = sl.page_of(next_key0 + kStreamWaves * kStep, kend);
  }
}

// ----------------------------------------------------------------- the prologue wave

// Lane (r4 = lane / 16, c16 = lane % 16) handles rows r = r4 + 4 * pass of the
// 16-row q' block (rows >= G are zero-filled) and, in lanes 0..15, the new
// key row.  prologue_issue only requests the rows; prologue_finish (after the
// streaming waves have queued their K/V loads) computes and writes to LDS
// what the streaming waves read after the next workgroup barrier.
template <bool BF16>
struct PrologueRegs {
  RawHalf<BF16> x[4];        // q rows r4 + 4 * pass (row min(r, G-1): rows >= G are discarded)
  RawHalf<BF16> gq, gk, y;   // norm weights (unused when NULL), the new key row
};

// Branch-free: every lane fetches valid rows, so no fetch is waited on here.
// The q rows and norm weights (prologue_issue_q) need only the group; the new
// key row (prologue_issue_k) needs the length and is fetched only by the
// workgroup whose range holds it, so that the others' q' waits on the q rows
// alone.
template <bool BF16>
__device__ __forceinline__ void prologue_issue_q(const DecodeParams& p, int b, int h, int lane, PrologueRegs<BF16>& pr) {
  constexpr int kElem = BF16 ? 2 : 4;
  const int r4 = lane >> 4, c16 = lane & 15;
  const int G = p.group;
#pragma unroll
  for (int ps = 0; ps < 4; ++ps) {
    const int r = min(4 * ps + r4, G - 1);
    const uint8_t* row = (const uint8_t*)p.q + ((int64_t)b * p.q_sb + (int64_t)(h * G + r) * p.q_sh) * kElem;
    pr.x[ps] = fetch_half_row<BF16>(row, c16);
  }
  pr.gq = fetch_half_row<BF16>(p.q_norm_w != nullptr ? p.q_norm_w : p.q, c16);
  pr.gk = fetch_half_row<BF16>(p.k_norm_w != nullptr ? p.k_norm_w : p.q, c16);
}
template <bool BF16>
__device__ __forceinline__ void prologue_issue_k(const uint8_t* krow, int lane, PrologueRegs<BF16>& pr) {
  pr.y = fetch_half_row<BF16>(krow, lane & 15);
}

template <bool BF16, class SM>
__device__ __forceinline__ void prologue_finish(const DecodeParams& p, SM& sm, double pos, int lane,
                                                bool rope, bool has_new, PrologueRegs<BF16>& pr) {
  const int r4 = lane >> 4, c16 = lane & 15;
  const int G = p.group;
  const bool qnorm = p.q_norm_w != nullptr, knorm = p.k_norm_w != nullptr;
  float gq[8], gk[8], q[4][8];
  unpack_half_row<BF16>(pr.gq, gq);
  unpack_half_row<BF16>(pr.gk, gk);
  if (rope) {
    // bf16: angle reduced to revolutions in double, hardware sin / cos;
    // f32: sin / cos in double
    const double inv = rope_inv_freq(lane, p.rope_log2_theta);
    if constexpr (BF16) rope_cos_sin_rev(pos, inv * 0.15915494309189535, sm.cs[lane][0], sm.cs[lane][1]);
    else rope_cos_sin_f64(pos, inv, sm.cs[lane][0], sm.cs[lane][1]);
    // the table is read back by other lanes of this wave only
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  }
#pragma unroll
  for (int ps = 0; ps < 4; ++ps) {
    const int r = 4 * ps + r4;
    float v[8];
    unpack_half_row<BF16>(pr.x[ps], v);
    prologue_row(v, c16, qnorm, gq, p.eps, rope, sm.cs);
    if (r >= G) {
#pragma unroll
      for (int j = 0; j < 8; ++j) v[j] = 0.f;
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) q[ps][j] = v[j];   // keep q' for the new-key score
    *(f32x4*)&sm.qp[r][4 * c16] = f32x4{v[0], v[1], v[2], v[3]};
    *(f32x4*)&sm.qp[r][64 + 4 * c16] = f32x4{v[4], v[5], v[6], v[7]};
    if constexpr (BF16) {
      float hv[8], lv[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        hv[j] = (float)(__bf16)v[j];
        lv[j] = v[j] - hv[j];
      }
      *(u32x2*)&sm.qh[r][4 * c16] = u32x2{pack_bf16x2(hv[0], hv[1]), pack_bf16x2(hv[2], hv[3])};
      *(u32x2*)&sm.qh[r][64 + 4 * c16] = u32x2{pack_bf16x2(hv[4], hv[5]), pack_bf16x2(hv[6], hv[7])};
      *(u32x2*)&sm.ql[r][4 * c16] = u32x2{pack_bf16x2(lv[0], lv[1]), pack_bf16x2(lv[2], lv[3])};
      *(u32x2*)&sm.ql[r][64 + 4 * c16] = u32x2{pack_bf16x2(lv[4], lv[5]), pack_bf16x2(lv[6], lv[7])};
    }
  }
  if (has_new) {
    float y[8];
    unpack_half_row<BF16>(pr.y, y);
    prologue_row(y, c16, knorm, gk, p.eps, rope, sm.cs);
    if (r4 == 0) {
      *(f32x4*)&sm.kn[4 * c16] = f32x4{y[0], y[1], y[2], y[3]};
      *(f32x4*)&sm.kn[64 + 4 * c16] = f32x4{y[4], y[5], y[6], y[7]};
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    const f32x4 ka = *(const f32x4*)&sm.kn[4 * c16], kb = *(const f32x4*)&sm.kn[64 + 4 * c16];
#pragma unroll
    for (int ps = 0; ps < 4; ++ps) {
      float d = 0.f;
#pragma unroll
      for (int j = 0; j < 4; ++j) d += q[ps][j] * ka[j] + q[ps][4 + j] * kb[j];
      d = sum16(d);
      if (c16 == 0) sm.snew[4 * ps + r4] = d * p.scale_log2;
    }
  }
}

// ----------------------------------------------------------------- partition kernel

__device__ __forceinline__ void write_zero_rows(const DecodeParams& p, int b, int h, int tid) {
  const int g = tid >> 4, d8 = (tid & 15) * 8;
  if (g >= p.group) return;
  uint8_t* o = (uint8_t*)p.out + ((int64_t)b * p.o_sb + (int64_t)(h * p.group + g) * p.o_sh) * (p.out_bf16 ? 2 : 4);
  if (p.out_bf16) {
    *(u32x4*)(o + 2 * d8) = u32x4{0, 0, 0, 0};
  } else {
    *(f32x4*)(o + 4 * d8) = f32x4{0.f, 0.f, 0.f, 0.f};
    *(f32x4*)(o + 4 * d8 + 16) = f32x4{0.f, 0.f, 0.f, 0.f};
  }
}

// The 4 wave states of one chunk held in LDS buffer `buf`, combined (ADR-0060
// section 4, in-workgroup level) for head g, dims d8 .. d8+7: the chunk's
// maximum M, sum l and unnormalised O.  The chunk holds at least one key, so
// M is finite.
template <class SM>
__device__ __forceinline__ void chunk_state(const SM& sm, int buf, int g, int d8, float& M, float& lt,
                                            float (&acc)[8]) {
  M = sm.mm[buf][0][g];
#pragma unroll
  for (int w = 1; w < kStreamWaves; ++w) M = fmaxf(M, sm.mm[buf][w][g]);
  lt = 0.f;
#pragma unroll
  for (int j = 0; j < 8; ++j) acc[j] = 0.f;
#pragma unroll
  for (int w = 0; w < kStreamWaves; ++w) {
    const float sc = fast_exp2(sm.mm[buf][w][g] - M);   // 0 for a wave that saw no key
    lt += sc * sm.ml[buf][w][g];
    const float* src = &sm.mo[buf][w][g][d8];
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[j] += sc * src[j];
  }
}

__device__ __forceinline__ void store_partial(const DecodeParams& p, int b, int hq, int wc, int d8, bool ml, float M,
                                              float lt, const float (&acc)[8]) {
  const int64_t slot = ((int64_t)b * p.num_q_heads + hq) * p.wpg + wc;
  float* wo = p.ws_o + slot * kHeadDim + d8;
  *(f32x4*)wo = f32x4{acc[0], acc[1], acc[2], acc[3]};
  *(f32x4*)(wo + 4) = f32x4{acc[4], acc[5], acc[6], acc[7]};
  if (ml) {
    p.ws_ml[2 * slot] = M;
    p.ws_ml[2 * slot + 1] = lt;
  }
}

// Merge of the 4 wave states of the workgroup's only chunk by `nthr` threads:
// thread t takes head t/16 (+ nthr/16, ...) and dims 8 (t%16) .. +7; the
// result is the workgroup's partial in slot wc (or, with a single chunk in
// the plan, the normalised output row).
template <class SM>
__device__ __forceinline__ void merge_chunk(const DecodeParams& p, const SM& sm, int buf, int b, int h, int wc,
                                            int t, int nthr) {
  const int G = p.group, d8 = (t & 15) * 8;
  for (int g = t >> 4; g < G; g += nthr >> 4) {
    float M, lt, acc[8];
    chunk_state(sm, buf, g, d8, M, lt, acc);
    const int hq = h * G + g;
    if (p.n_split == 1) {
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
      store_partial(p, b, hq, wc, d8, (t & 15) == 0, M, lt, acc);
    }
  }
}

// Running log-sum-exp merge of the chunks a workgroup sweeps, kept by the 64
// lanes of the prologue wave: lane t holds heads t/16 + 4k (k < 4) at dims
// 8 (t%16) .. +7.  Seeded (-inf, 0, 0).
struct RunMerge {
  float m[4], l[4];
  float o[4][8];
};

template <class SM>
__device__ __forceinline__ void fold_chunk(const DecodeParams& p, const SM& sm, int buf, int lane,
                                           RunMerge& r) {
  const int d8 = (lane & 15) * 8;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const int g = (lane >> 4) + 4 * k;
    if (g < p.group) {
      float M, lt, acc[8];
      chunk_state(sm, buf, g, d8, M, lt, acc);
      const float mn = fmaxf(r.m[k], M);
      const float a = fast_exp2(r.m[k] - mn), c = fast_exp2(M - mn);   // a = 0 on the first chunk
      r.l[k] = a * r.l[k] + c * lt;
#pragma unroll
      for (int j = 0; j < 8; ++j) r.o[k][j] = a * r.o[k][j] + c * acc[j];
      r.m[k] = mn;
    }
  }
}

__device__ __forceinline__ void store_run(const DecodeParams& p, const RunMerge& r, int b, int h, int wc, int lane) {
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const int g = (lane >> 4) + 4 * k;
    if (g < p.group) store_partial(p, b, h * p.group + g, wc, (lane & 15) * 8, (lane & 15) == 0, r.m[k], r.l[k], r.o[k]);
  }
}

// A workgroup sweeps `cpw` consecutive chunks of one (b, KV head) group and
// writes one partial: the log-sum-exp merge of its chunks.  The streaming
// waves load continuously across chunk boundaries; at the end of each chunk
// they leave their states in one of two LDS buffers and meet the prologue
// wave at a barrier, after which the prologue wave folds that chunk into its
// running merge while they sweep the next one.  (Chunks are multiples of 32
// keys whenever cpw > 1, so no step spans two chunks.)
// Two waves per SIMD at most (one workgroup of 5 waves per compute unit): no
// register spills, which matters most for long sweeps (a spill reload would
// queue behind the wave's in-flight K/V loads).
// Row j of the (sequence b, KV head h) K cache: contiguous, or through the
// block table (page stride k_sb).
template <bool PAGED>
__device__ __forceinline__ const uint8_t* k_row(const DecodeParams& p, int b, int h, int j, int elem) {
  if constexpr (PAGED) {
    const int page = p.block_table[(int64_t)b * p.max_blocks + (j >> p.block_log2)];
    return (const uint8_t*)p.k +
           ((int64_t)page * p.k_sb + (int64_t)h * p.k_sh + (int64_t)(j & ((1 << p.block_log2) - 1)) * p.k_ss) * elem;
  } else {
    return (const uint8_t*)p.k + ((int64_t)b * p.k_sb + (int64_t)h * p.k_sh + (int64_t)j * p.k_ss) * elem;
  }
}

// Inclusive prefix sum over the 64 lanes of a wave: shifts by 1, 2, 4 and 8
// lanes inside each 16-lane row (DPP row_shr, zeros shifted in), then the
// last lane of rows 0 and 2 added to rows 1 and 3 (row_bcast:15), then lane
// 31 to rows 2 and 3 (row_bcast:31).
template <int CTRL, int ROWS>
__device__ __forceinline__ int dpp_int(int v) {
  return __builtin_amdgcn_update_dpp(0, v, CTRL, ROWS, 0xF, false);
}
__device__ __forceinline__ int wave_prefix_sum(int v) {
  v += dpp_int<0x111, 0xF>(v);
  v += dpp_int<0x112, 0xF>(v);
  v += dpp_int<0x114, 0xF>(v);
  v += dpp_int<0x118, 0xF>(v);
  v += dpp_int<0x142, 0xA>(v);
  v += dpp_int<0x143, 0xC>(v);
  return v;
}

// Workgroup -> (group, its workgroup wc, the group's clamped length and its
// sequence's position) for a batch of several sequences, with every workgroup whose key range holds keys
// ahead of those past their sequence's end.  The lengths are device data, so
// the grid still covers every range (ceil(n_split / cpw) per group); a
// workgroup reads the lengths of the groups it may serve and finds its range
// by a prefix sum over their live-workgroup counts ceil(L / (split cpw)), one
// for L = 0 (it writes that group's zero rows when the plan is unsplit).  When
// the group count is a multiple of 8, XCD x serves groups x, x + 8, ... in
// that order (workgroup x + 8 s is the s-th of XCD x), so a group's partials
// stay in one L2 for the merge; otherwise groups are served in order.  Every
// wave of a workgroup reads the same lengths and reaches the same answer;
// false for the workgroups past the live ones, which return without touching
// memory.  The positions come with the lengths (vector loads: a scalar load
// issued behind a compute unit's K/V stream returns late).  (A batch of one
// maps its workgroups statically, without the lengths.)
__device__ __forceinline__ bool live_slot(const DecodeParams& p, int lane, int& grp, int& wc, int& len, int& posv) {
  const int groups = p.batch * p.num_kv_heads;
  const int keys = p.split * p.cpw;   // keys per workgroup
  const bool by_xcd = groups % kXcds == 0;
  const int first = by_xcd ? (int)(blockIdx.x % kXcds) : 0, stride = by_xcd ? kXcds : 1;
  const int n = by_xcd ? groups / kXcds : groups;
  int s = by_xcd ? (int)(blockIdx.x / kXcds) : (int)blockIdx.x;
  for (int base = 0; base < n; base += 64) {
    const int j = base + lane;
    int Lj = 0, cnt = 0, Pj = 0;
    if (j < n) {
      Lj = p.seq_lens[(first + stride * j) / p.num_kv_heads];
      Pj = p.positions[(first + stride * j) / p.num_kv_heads];
      Lj = Lj < 0 ? 0 : (Lj > p.max_seq ? p.max_seq : Lj);
      cnt = Lj == 0 ? 1 : (Lj + keys - 1) / keys;
    }
    const int incl = wave_prefix_sum(cnt);
    const unsigned long long hit = __ballot(j < n && s < incl);
    if (hit != 0) {
      const int l = (int)__builtin_ctzll(hit);   // the first lane whose prefix passes s
      const int excl = __builtin_amdgcn_readlane(incl - cnt, l);
      const int w = s - excl;
      if (base + l >= n || w < 0 || w >= __builtin_amdgcn_readlane(cnt, l)) return false;   // never taken
      grp = first + stride * (base + l);
      wc = w;
      len = __builtin_amdgcn_readlane(Lj, l);
      posv = __builtin_amdgcn_readlane(Pj, l);
      return true;
    }
    s -= __builtin_amdgcn_readlane(incl, 63);
  }
  return false;
}

// PW: a dedicated prologue wave beside the 4 streaming waves (any plan);
// otherwise the 4-wave form for single-chunk workgroups (cpw = 1), whose
// streaming wave 0 runs the prologue.
template <bool BF16, bool PAGED, bool PW>
__global__ __launch_bounds__(PW ? kThreads : kThreads4, BF16 ? 2 : 1) void decode_partition_kernel(const DecodeParams p) {
  using Step = typename std::conditional<BF16, StepBF16, StepF32>::type;
  using QFrag = typename std::conditional<BF16, QFragBF16, QFragF32>::type;
  constexpr int kElem = BF16 ? 2 : 4;
  constexpr int kPW = PW ? kPrologueWave : 0;        // the wave that runs the prologue
  constexpr int kNT = PW ? kThreads : kThreads4;

  __shared__ DecodeSmemT<PW ? 2 : 1> sm;
#ifdef GQA_TIMELINE
  __shared__ uint64_t tl[kTimelineSlots];
#endif

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform branches
  const int n16 = lane & 15, q4 = lane >> 4;
  const bool direct = p.n_split == 1;
  GQA_STAMP(wave == kPW && lane == 0, 0);   // entry

  // ---- workgroup -> (group = (b, h), chunks cf .. cf + cpw - 1)
  int grp, wc, L, posv = 0;
  PrologueRegs<BF16> pr;
  if (p.batch == 1) {
    // one length for every group: a static map (the workgroups of a group
    // consecutive, on one XCD when the group count allows), so the prologue
    // wave requests the q rows and norm weights while the length is read
    const int groups = p.num_kv_heads;
    const bool by_xcd = groups % kXcds == 0;
    const int s = by_xcd ? (int)(blockIdx.x / kXcds) : (int)blockIdx.x;
    grp = (by_xcd ? (int)(blockIdx.x % kXcds) : 0) + (by_xcd ? kXcds : 1) * (s / p.wpg);
    wc = s % p.wpg;
    if (wave == kPW) prologue_issue_q<BF16>(p, 0, grp, lane, pr);
    L = p.seq_lens[0];
    posv = p.positions[0];   // with the length: issued after it, it would queue behind the K/V stream
    L = L < 0 ? 0 : (L > p.max_seq ? p.max_seq : L);
    if (wc > 0 && wc * p.split * p.cpw >= L) return;   // past the sequence (wc = 0 writes an empty one's zero rows)
  } else {
    if (!live_slot(p, lane, grp, wc, L, posv)) return;   // past every live range: nothing to do
  }
  GQA_STAMP(wave == kPW && lane == 0, 1);   // length known
  const int b = grp / p.num_kv_heads, h = grp % p.num_kv_heads;
  const int cf = wc * p.cpw;
  const int c0 = cf * p.split;
  const int cap = min(min(cf + p.cpw, p.n_split) * p.split, p.max_seq);   // static end of the range

  Slab<PAGED> sl;
  if constexpr (PAGED) {   // head h inside every page; pages through this sequence's block-table row
    sl.kb = (const uint8_t*)p.k + (int64_t)h * p.k_sh * kElem;
    sl.vb = (const uint8_t*)p.v + (int64_t)h * p.v_sh * kElem;
    sl.bt = p.block_table + (int64_t)b * p.max_blocks;
    sl.log2bs = p.block_log2;
    sl.kpage = p.k_sb * kElem;
    sl.vpage = p.v_sb * kElem;
  } else {
    sl.kb = (const uint8_t*)p.k + ((int64_t)b * p.k_sb + (int64_t)h * p.k_sh) * kElem;
    sl.vb = (const uint8_t*)p.v + ((int64_t)b * p.v_sb + (int64_t)h * p.v_sh) * kElem;
  }
  sl.kss = (uint32_t)(p.k_ss * kElem);
  sl.vss = (uint32_t)(p.v_ss * kElem);
  if constexpr (BF16) {
    sl.klane = (uint32_t)n16 * sl.kss + 16u * q4;          // K row n16, dims 32*kb + 8*q4 ..
    sl.vlane = (uint32_t)(4 * q4) * sl.vss + 16u * n16;    // V rows 4*q4 + .., dims 8*n16 ..
  } else {
    sl.klane = (uint32_t)n16 * sl.kss + 128u * q4;
    sl.vlane = (uint32_t)(4 * q4) * sl.vss + 32u * n16;
  }

  // ---- the prologue wave requests its rows, then the streaming waves queue
  //      their first K/V steps behind them (one memory queue per compute unit)
  const bool stream = wave < kStreamWaves;
  const bool rope = p.rope_theta > 0.0;
  const double pos = rope ? (double)posv : 0.0;
  const int c1 = min(cap, L);
  const bool has_new = (rope || p.k_norm_w != nullptr) && c0 < L && c1 == L;   // range holds slot L-1
  const int kn = has_new ? L - 1 : -1;
  if (wave == kPW && c0 < L) {
    if (p.batch != 1) prologue_issue_q<BF16>(p, b, h, lane, pr);
    if (has_new) prologue_issue_k<BF16>(k_row<PAGED>(p, b, h, kn, kElem), lane, pr);
  }
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");   // keeps the loads above on this side
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

  if (c0 >= L) {     // no keys in this range: no partial, no arrival
    if (cf == 0 && direct) write_zero_rows(p, b, h, tid);   // L == 0: all-zero output rows
    return;
  }
  const int nsteps = (c1 - c0 + kStep - 1) / kStep;
  const int nchunks = (c1 - c0 + p.split - 1) / p.split;        // chunks of this range holding keys
  const int spc = nchunks == 1 ? nsteps : p.split / kStep;      // steps per chunk
  int s = wave;
  Step A;
  int page = 0;   // paged: the page of this wave's next step
  if (stream && s < nsteps) {
    load_step(A, sl, c0 + s * kStep, c1, n16, q4, sl.page_of(c0 + s * kStep, c1));
    page = sl.page_of(c0 + (s + kStreamWaves) * kStep, c1);
  }
  GQA_STAMP(wave == 0 && lane == 0, 2);   // first K/V step requested
  if (wave == kPW) prologue_finish<BF16>(p, sm, pos, lane, rope, has_new, pr);
  GQA_STAMP(wave == kPW && lane == 0, 3);   // prologue done
  __syncthreads();   // q', the new-key score and the tables are in LDS
  GQA_STAMP(wave == 0 && lane == 0, 4);   // sweep starts

  if (stream) {
    QFrag qf;
    load_qfrag(qf, sm, n16, q4);
    for (int j = 0; j < nchunks; ++j) {
      RunState rs;
#pragma unroll
      for (int T = 0; T < 8; ++T) rs.o[T] = f32x4{0.f, 0.f, 0.f, 0.f};
      rs.m = -INFINITY;
      rs.l = 0.f;
      // one step buffer per wave, refilled in place: the next step's K is in
      // flight during this step's softmax and P V, its V during the next QK^T
      const int s_end = min(nsteps, (j + 1) * spc);
      while (s < s_end) {
        const int next = c0 + (s + kStreamWaves) * kStep;
        if constexpr (BF16) {
          if (next >= c1) {   // this wave's last step of the range: no refill
            sweep_step<kNoRefill>(A, qf, sm.snew, kn, rs, p.scale_log2, c0 + s * kStep, c1, next, sl, n16, q4, page);
            s += kStreamWaves;
            break;
          }
          sweep_step<kRefill>(A, qf, sm.snew, kn, rs, p.scale_log2, c0 + s * kStep, c1, next, sl, n16, q4, page);
        } else {
          sweep_step<kRefillIfMore>(A, qf, sm.snew, kn, rs, p.scale_log2, c0 + s * kStep, c1, next, sl, n16, q4, page);
        }
        s += kStreamWaves;
      }
      // ---- this wave's state of chunk j into LDS buffer j % 2 (the only one
      //      in the 4-wave form, whose workgroups hold one chunk)
      const int buf = PW ? (j & 1) : 0;
      rs.l = sum_xor32(sum_xor16(rs.l));
      if (q4 == 0) {
        sm.mm[buf][wave][n16] = rs.m;
        sm.ml[buf][wave][n16] = rs.l;
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        float* dst = &sm.mo[buf][wave][n16][(4 * q4 + i) * 8];
        *(f32x4*)dst = f32x4{rs.o[0][i], rs.o[1][i], rs.o[2][i], rs.o[3][i]};
        *(f32x4*)(dst + 4) = f32x4{rs.o[4][i], rs.o[5][i], rs.o[6][i], rs.o[7][i]};
      }
      __syncthreads();
    }
    GQA_STAMP(wave == 0 && lane == 0, 5);   // sweep done
  } else if constexpr (PW) {
    // the prologue wave folds chunk j while the streaming waves sweep chunk j+1,
    // then the last chunk, and stores the workgroup's partial
    RunMerge run;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      run.m[k] = -INFINITY;
      run.l[k] = 0.f;
#pragma unroll
      for (int j = 0; j < 8; ++j) run.o[k][j] = 0.f;
    }
    for (int j = 0; j + 1 < nchunks; ++j) {
      __syncthreads();
      fold_chunk(p, sm, j & 1, lane, run);
    }
    __syncthreads();
    if (nchunks > 1) {
      fold_chunk(p, sm, (nchunks - 1) & 1, lane, run);
      store_run(p, run, b, h, wc, lane);
    }
  }
  // ---- the new key's transformed row replaces the raw one in its cache slot:
  //      every read of that row (the prologue's and the streaming waves' step
  //      holding it) is complete, and no other workgroup reads it
  if (p.write_new_k && has_new && wave == kPW && lane < 32) {
    uint8_t* row = (uint8_t*)k_row<PAGED>(p, b, h, kn, kElem);
    const f32x4 y = *(const f32x4*)&sm.kn[4 * lane];
    if (BF16) *(u32x2*)(row + 8 * lane) = u32x2{pack_bf16x2(y[0], y[1]), pack_bf16x2(y[2], y[3])};
    else *(f32x4*)(row + 16 * lane) = y;
  }
  // ---- a single chunk: every thread of the workgroup merges its wave states
  if (nchunks == 1) merge_chunk(p, sm, 0, b, h, wc, tid, kNT);
#ifdef GQA_TIMELINE
  GQA_STAMP(tid == 0, 6);   // partial (or output rows) stored
  __syncthreads();
  if (tid < kTimelineSlots && blockIdx.x < kTimelineBlocks) g_timeline[blockIdx.x * kTimelineSlots + tid] = tl[tid];
#endif
}

// ----------------------------------------------------------------- merge kernel
// One workgroup per (q head, sequence): out = sum_c 2^(m_c - M) O_c / sum_c 2^(m_c - M) l_c
// over the partials of the n = ceil(L / (cpw T)) partition workgroups that
// hold keys (ADR-0060 section 4).  Thread
// (group sg, dims 4*d4 .. 4*d4+3) folds chunks sg, sg + 4, ... with a running
// maximum, kMergeUnroll chunks per batch of loads; the 4 group states are then
// merged through LDS.

constexpr int kMergeThreads = 128;
constexpr int kMergeGroups = kMergeThreads / 32;
constexpr int kMergeUnroll = 8;

__global__ __launch_bounds__(kMergeThreads) void decode_merge_kernel(const DecodeParams p) {
  __shared__ __attribute__((aligned(16))) float racc[kMergeGroups][kHeadDim];
  __shared__ float rm[kMergeGroups], rl[kMergeGroups];

  // workgroup -> (b, q head hq): on the XCD that ran the partition workgroups
  // of its (b, KV head) group when the group count allows it (partials in L2)
  const int G = p.group, groups = p.batch * p.num_kv_heads;
  const int bid = blockIdx.x, tid = threadIdx.x;
  int b, hq;
  if (groups % kXcds == 0) {
    const int slot = bid / kXcds;
    const int grp = bid % kXcds + kXcds * (slot / G);
    b = grp / p.num_kv_heads;
    hq = (grp % p.num_kv_heads) * G + slot % G;
  } else {
    b = bid / p.num_q_heads;
    hq = bid % p.num_q_heads;
  }
  int L = p.seq_lens[b];
  L = L < 0 ? 0 : (L > p.max_seq ? p.max_seq : L);
  const int64_t span = (int64_t)p.cpw * p.split;
  const int n = (int)((L + span - 1) / span);   // partition workgroups that wrote a partial
  uint8_t* o = (uint8_t*)p.out + ((int64_t)b * p.o_sb + (int64_t)hq * p.o_sh) * (p.out_bf16 ? 2 : 4);
  if (n == 0) {
    if (tid < 32) {
      if (p.out_bf16) *(u32x2*)(o + 8 * tid) = u32x2{0, 0};
      else *(f32x4*)(o + 16 * tid) = f32x4{0.f, 0.f, 0.f, 0.f};
    }
    return;
  }
  const int64_t slot0 = ((int64_t)b * p.num_q_heads + hq) * p.wpg;
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

template <bool BF16>
hipError_t launch_partition(const DecodeParams& p, hipStream_t stream) {
  const int wpg = (p.n_split + p.cpw - 1) / p.cpw;
  const dim3 grid(wpg * p.num_kv_heads * p.batch);
  if constexpr (BF16) {
    if (p.cpw == 1 && grid.x >= kMany4) {   // many single-chunk workgroups: two per compute unit
      if (p.block_table != nullptr)
        return launch_kernel(decode_partition_kernel<BF16, true, false>, grid, dim3(kThreads4), stream, p);
      return launch_kernel(decode_partition_kernel<BF16, false, false>, grid, dim3(kThreads4), stream, p);
    }
  }
  if (p.block_table != nullptr)
    return launch_kernel(decode_partition_kernel<BF16, true, true>, grid, dim3(kThreads), stream, p);
  return launch_kernel(decode_partition_kernel<BF16, false, true>, grid, dim3(kThreads), stream, p);
}

}  // namespace

hipError_t launch_decode_partition(const DecodeParams& p, bool in_bf16, hipStream_t stream) {
  return in_bf16 ? launch_partition<true>(p, stream) : launch_partition<false>(p, stream);
}

hipError_t launch_decode_merge(const DecodeParams& p, hipStream_t stream) {
  if (p.n_split == 1) return hipSuccess;
  return launch_kernel(decode_merge_kernel, dim3(p.num_q_heads * p.batch), dim3(kMergeThreads), stream, p);
}

}  // namespace gqa

#ifdef GQA_TIMELINE
// include/gqa_timeline.h: exported by the measurement build only.
namespace gqa {
hipError_t timeline_attn_clear(const uint64_t* zeros, size_t bytes);   // prefill_phased.hip
hipError_t timeline_attn_read(uint64_t* host, size_t bytes);
}  // namespace gqa

extern "C" int32_t gqa_timeline_clear(void) {
  static uint64_t zeros[GQA_TIMELINE_BLOCKS * GQA_TIMELINE_SLOTS];   // zero-initialised
  hipError_t e = hipMemcpyToSymbol(HIP_SYMBOL(gqa::g_timeline), zeros, sizeof(zeros));
  if (e == hipSuccess) e = gqa::timeline_attn_clear(zeros, sizeof(zeros));
  return (int32_t)e;
}

extern "C" int32_t gqa_timeline_read(int32_t kernel, uint64_t* host, size_t words) {
  if (host == nullptr || words > (size_t)GQA_TIMELINE_BLOCKS * GQA_TIMELINE_SLOTS) return 1;
  if (kernel == GQA_TIMELINE_DECODE)
    return (int32_t)hipMemcpyFromSymbol(host, HIP_SYMBOL(gqa::g_timeline), words * sizeof(uint64_t));
  if (kernel == GQA_TIMELINE_PREFILL) return (int32_t)gqa::timeline_attn_read(host, words * sizeof(uint64_t));
  return 1;
}

extern "C" int32_t gqa_timeline_clock_khz(int32_t* khz) {
  if (khz == nullptr) return 1;
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e == hipSuccess) e = hipDeviceGetAttribute(khz, hipDeviceAttributeWallClockRate, dev);
  return (int32_t)e;
}
#endif
