// Internal header of the gfx950 GQA attention library: launch parameter
// structs, launcher declarations and small device helpers shared by the
// decode and prefill kernels.  Not part of the public ABI (include/gqa_attn.h).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gqa {

constexpr int kHeadDim = 128;

// ----------------------------------------------------------------- params

struct DecodeParams {
  const void* q;
  const void* k;
  const void* v;
  const int32_t* seq_lens;
  const int32_t* positions;
  const void* q_norm_w;   // may be null: no RMSNorm on q
  const void* k_norm_w;   // may be null: no RMSNorm on the new key row
  void* out;
  float* ws_o;            // [B][Hq][wpg][128] unnormalised partial O, one per partition workgroup
  float* ws_ml;           // [B][Hq][wpg][2]   (m in log2 units, l)
  int64_t q_sb, q_sh;     // element strides
  int64_t k_sb, k_sh, k_ss;
  int64_t v_sb, v_sh, v_ss;
  int64_t o_sb, o_sh;
  int32_t batch, num_q_heads, num_kv_heads, group, max_seq;
  int32_t split, n_split;
  int32_t cpw;            // chunks swept by one partition workgroup (1, or more when split % 32 == 0)
  int32_t wpg;            // partition workgroups (= partial slots) per (b, KV head): ceil(n_split / cpw)
  int32_t out_bf16;
  int32_t write_new_k;    // store the new key's transformed row back into the cache slot
  const int32_t* block_table;  // paged caches: [B][max_blocks] page of each block of rows (null: contiguous)
  int32_t block_log2;     // paged: log2(rows per page)
  int32_t max_blocks;     // paged: row length of block_table
  float eps;
  float scale_log2;       // softmax scale * log2(e): scores live in the log2 domain
  double rope_theta;      // <= 0: RoPE off
  double rope_log2_theta; // log2(rope_theta) when RoPE is on
};

struct PrefillParams {
  const void* q;
  const void* k;
  const void* v;
  const int32_t* seq_lens;
  const int32_t* positions;
  const void* q_norm_w;
  const void* k_norm_w;
  void* out;
  int64_t q_sb, q_sh, q_ss;
  int64_t k_sb, k_sh, k_ss;
  int64_t v_sb, v_sh, v_ss;
  int64_t o_sb, o_sh, o_ss;
  int32_t batch, num_q_heads, num_kv_heads, group, max_seq;
  int32_t causal;
  int32_t out_bf16;
  const int32_t* past_lens;  // chunked prefill: keys already in the cache per sequence (null: none)
  const int32_t* block_table;  // paged caches: [B][max_blocks] page of each block of rows (null: contiguous)
  int32_t block_log2;     // paged: log2(rows per page)
  int32_t max_blocks;     // paged: row length of block_table
  int32_t max_chunk;      // query / output rows per sequence (max_seq for a plain prefill)
  int32_t write_k_cache;  // two-phase: store each new key's post-prologue row (bf16) over its raw row
  int32_t span_tiles;     // two-phase: at most this many 32-key tiles per attention workgroup
  int32_t n_spans;        // two-phase: key spans per query block in the grid (1: no split)
  uint32_t* counters;     // two-phase, n_spans > 1: arrivals per (b, q head, query block)
  int32_t n_counters;
  float* partials;        // two-phase, n_spans > 1: (m, l, O) of each (b, q head, query block, span)
  int32_t heads_per_wg;   // HC: query heads of one KV head batched in a workgroup
  int32_t block_q;        // BQ: query tokens per workgroup (multiple of 32)
  int32_t n_qblocks;      // ceil(max_seq / BQ)
  float eps;
  float scale_log2;
  double rope_theta;
  double rope_log2_theta;
};

// Launch of `kernel` with its arguments; returns the status of this launch
// (hipLaunchKernel), not a sticky error an earlier HIP call of the process
// may have left behind.
template <typename... Args>
inline hipError_t launch_kernel(void (*kernel)(Args...), dim3 grid, dim3 block, hipStream_t stream, Args... args) {
  void* ptrs[] = {(void*)&args...};
  return hipLaunchKernel((const void*)kernel, grid, block, ptrs, 0, stream);
}

// Launchers (return the status of their launches).
hipError_t launch_decode_partition(const DecodeParams& p, bool in_bf16, hipStream_t stream);
hipError_t launch_decode_merge(const DecodeParams& p, hipStream_t stream);
hipError_t launch_prefill_fused(const PrefillParams& p, hipStream_t stream);
// Phases of the two-phase prefill: the key prologue into the workspace, then
// attention over it.
constexpr int kPhaseKeys = 1;
constexpr int kPhaseAttend = 2;
hipError_t launch_prefill_phased(const PrefillParams& p, void* workspace, hipStream_t stream,
                                 int phases = kPhaseKeys | kPhaseAttend);
// Bytes of the two-phase prefill workspace, for a plain prefill (max_chunk =
// max_seq) and a chunked one (max_chunk <= max_seq) alike.
size_t prefill_workspace_bytes(int batch, int num_q_heads, int num_kv_heads, int max_seq, int max_chunk, bool causal);

// Prefill workgroups hold HC * BQ / 32 waves of 32 query rows, at most this many.
constexpr int kPrefillMaxWaves = 10;

// ----------------------------------------------------------------- device helpers

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;
typedef __attribute__((ext_vector_type(8))) _Float16 f16x8;
typedef __attribute__((ext_vector_type(2))) _Float16 f16x2;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(2))) float f32x2;
typedef __attribute__((ext_vector_type(16))) float f32x16;
typedef __attribute__((ext_vector_type(4))) uint32_t u32x4;
typedef __attribute__((ext_vector_type(2))) uint32_t u32x2;

__device__ __forceinline__ float bf16lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// Two floats -> packed bf16 pair (round to nearest even; v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  bf16x2 v;
  v[0] = (__bf16)lo;
  v[1] = (__bf16)hi;
  return __builtin_bit_cast(uint32_t, v);
}

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

// Two f32 to packed fp16 (round to nearest even; beyond +-65504 -> +-inf).
__device__ __forceinline__ uint32_t pack_f16x2(float lo, float hi) {
  const f16x2 v = {(_Float16)lo, (_Float16)hi};
  return __builtin_bit_cast(uint32_t, v);
}

__device__ __forceinline__ f16x8 as_f16x8(u32x4 v) { return __builtin_bit_cast(f16x8, v); }

// Largest finite fp16 magnitude.
constexpr float kF16Max = 65504.0f;

// x clamped to [-65504, 65504]; NaN stays NaN (IEEE maximum / minimum
// propagate it, unlike fmaxf / fminf).
__device__ __forceinline__ float clamp_f16_range(float x) {
  return __builtin_elementwise_minimum(__builtin_elementwise_maximum(x, -kF16Max), kF16Max);
}

// Two f32 to packed fp16, saturating: magnitudes beyond 65504 become +-65504
// instead of +-inf (round to nearest even inside the range).  Used for the
// prefill operands q', k' and v, whose range is the caller's.
__device__ __forceinline__ uint32_t pack_f16x2_sat(float lo, float hi) {
  return pack_f16x2(clamp_f16_range(lo), clamp_f16_range(hi));
}

// The fp16 saturation of pack_f16x2_sat applied after an unsaturated
// conversion: a half that became +-inf (|x| >= 65520 rounds there) is set to
// +-65504, which is what converting the clamped value gives; finite halves
// and NaN are unchanged.
__device__ __forceinline__ uint32_t saturate_inf_f16x2(uint32_t w) {
  const uint32_t lo = w & 0xffffu, hi = w >> 16;
  return (((lo & 0x7fffu) == 0x7c00u) ? lo - 1u : lo) | ((((hi & 0x7fffu) == 0x7c00u) ? hi - 1u : hi) << 16);
}

// Element e (0..7) of 8 packed bf16 held in 4 dwords, as float.
__device__ __forceinline__ float bf16_elem(const u32x4& v, int e) {
  uint32_t w = v[e >> 1];
  return (e & 1) ? bf16hi(w) : bf16lo(w);
}

// Low / high bf16 halves of two dwords combined into one dword:
// (lo of a, lo of b) and (hi of a, hi of b).
__device__ __forceinline__ uint32_t pair_lo(uint32_t a, uint32_t b) { return (a & 0xffffu) | (b << 16); }
__device__ __forceinline__ uint32_t pair_hi(uint32_t a, uint32_t b) { return (a >> 16) | (b & 0xffff0000u); }

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// ---- cross-lane reductions without LDS: DPP within 16-lane rows,
//      v_permlane16_swap / v_permlane32_swap across rows (gfx950)

template <int CTRL>
__device__ __forceinline__ float dpp_mov(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}

// Sum over each group of 8 lanes 8k .. 8k+7 (result in all 8).
__device__ __forceinline__ float sum8(float v) {
  v += dpp_mov<0xB1>(v);    // quad_perm [1,0,3,2]: lane ^ 1
  v += dpp_mov<0x4E>(v);    // quad_perm [2,3,0,1]: lane ^ 2
  v += dpp_mov<0x141>(v);   // row_half_mirror: the other quad of the 8
  return v;
}

// Sum over each 16-lane row.
__device__ __forceinline__ float sum16(float v) {
  v = sum8(v);
  return v + dpp_mov<0x140>(v);   // row_mirror: the other 8 of the row
}

// {v[lane], v[lane ^ 16]} and {v[lane], v[lane ^ 32]}, in the same order in both lanes.
__device__ __forceinline__ void pair_xor16(float v, float& a, float& b) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  a = __uint_as_float(r[0]);
  b = __uint_as_float(r[1]);
}
__device__ __forceinline__ void pair_xor32(float v, float& a, float& b) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  a = __uint_as_float(r[0]);
  b = __uint_as_float(r[1]);
}
__device__ __forceinline__ float max_xor16(float v) { float a, b; pair_xor16(v, a, b); return fmaxf(a, b); }
__device__ __forceinline__ float max_xor32(float v) { float a, b; pair_xor32(v, a, b); return fmaxf(a, b); }
__device__ __forceinline__ float sum_xor16(float v) { float a, b; pair_xor16(v, a, b); return a + b; }
__device__ __forceinline__ float sum_xor32(float v) { float a, b; pair_xor32(v, a, b); return a + b; }

// RoPE inverse frequency theta^(-2i/128) = 2^(-(2i/128) log2 theta), in double.
__device__ __forceinline__ double rope_inv_freq(int i, double log2_theta) {
  return exp2(-(double)(2 * i) / (double)kHeadDim * log2_theta);
}

// cos / sin of the RoPE angle pos * inv, formed and evaluated in double
// precision.  Used where only a few angles are needed.
__device__ __forceinline__ void rope_cos_sin_f64(double pos, double inv, float& c, float& s) {
  double sn, cn;
  sincos(pos * inv, &sn, &cn);
  c = (float)cn;
  s = (float)sn;
}

// cos / sin of the angle pos * inv where inv_rev = inv / (2 pi): the product
// and its reduction to [0, 1) revolutions (v_fract_f64) are done in double,
// the final sin / cos by the hardware instructions (which take revolutions).
__device__ __forceinline__ void rope_cos_sin_rev(double pos, double inv_rev, float& c, float& s) {
  const float rf = (float)__builtin_amdgcn_fract(pos * inv_rev);
  s = __builtin_amdgcn_sinf(rf);
  c = __builtin_amdgcn_cosf(rf);
}

}  // namespace gqa
