// C ABI of the gfx950 GQA attention library: argument validation (all on the
// host, before any HIP call), the split-KV plan, workspace sizing and the
// kernel launches.  The contract of every entry point is in include/gqa_attn.h.
#include <math.h>
#include <stdint.h>

#include <mutex>

#include "../../include/gqa_attn.h"
#include "common.hpp"

namespace {

constexpr int kGridYZMax = 65535;

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }
bool stride_ok(int64_t s, int elem) { return s >= 0 && ((s * elem) & 15) == 0; }
int elem_size(int32_t dt) { return dt == GQA_BF16 ? 2 : 4; }
bool dtype_ok(int32_t dt) { return dt == GQA_F32 || dt == GQA_BF16; }

float resolve_scale_log2(float scale) {
  const double s = scale > 0.f ? (double)scale : 1.0 / sqrt((double)GQA_ATTN_HEAD_DIM);
  return (float)(s * 1.4426950408889634);   // scores are kept in log2 units
}

// Shape / dtype / stride checks that need no pointer.
gqa_status check_decode_desc(const gqa_decode_desc* d) {
  if (d == nullptr) return GQA_ERR_NULL;
  if (d->batch < 1 || d->num_q_heads < 1 || d->num_kv_heads < 1 || d->max_seq < 1) return GQA_ERR_SHAPE;
  if (d->batch > kGridYZMax || d->num_kv_heads > kGridYZMax) return GQA_ERR_SHAPE;
  if ((int64_t)d->batch * d->num_q_heads > INT32_MAX) return GQA_ERR_SHAPE;   // merge grid
  if (d->num_q_heads % d->num_kv_heads != 0) return GQA_ERR_SHAPE;
  if (d->kv_split_tokens < 0) return GQA_ERR_SHAPE;
  if (d->block_size != 0) {   // paged: a power of two >= 32 rows per page, whole pages
    if (d->block_size < 32 || (d->block_size & (d->block_size - 1)) != 0 || d->max_seq % d->block_size != 0)
      return GQA_ERR_SHAPE;
  }
  if (d->head_dim != GQA_ATTN_HEAD_DIM) return GQA_ERR_UNSUPPORTED;
  if (d->num_q_heads / d->num_kv_heads > GQA_ATTN_MAX_GROUP) return GQA_ERR_UNSUPPORTED;
  if (!dtype_ok(d->in_dtype) || !dtype_ok(d->out_dtype)) return GQA_ERR_UNSUPPORTED;
  const int ei = elem_size(d->in_dtype), eo = elem_size(d->out_dtype);
  if (d->q_stride_b < 0 || d->q_stride_h < 0 || d->k_stride_b < 0 || d->k_stride_h < 0 || d->k_stride_s < 0 ||
      d->v_stride_b < 0 || d->v_stride_h < 0 || d->v_stride_s < 0 || d->out_stride_b < 0 || d->out_stride_h < 0)
    return GQA_ERR_SHAPE;
  // decode addresses one (b, KV head) cache slab with 32-bit byte offsets
  if ((int64_t)d->max_seq * d->k_stride_s * ei + 512 > ((int64_t)1 << 32) ||
      (int64_t)d->max_seq * d->v_stride_s * ei + 512 > ((int64_t)1 << 32))
    return GQA_ERR_UNSUPPORTED;
  if (!stride_ok(d->q_stride_b, ei) || !stride_ok(d->q_stride_h, ei) || !stride_ok(d->k_stride_b, ei) ||
      !stride_ok(d->k_stride_h, ei) || !stride_ok(d->k_stride_s, ei) || !stride_ok(d->v_stride_b, ei) ||
      !stride_ok(d->v_stride_h, ei) || !stride_ok(d->v_stride_s, ei) || !stride_ok(d->out_stride_b, eo) ||
      !stride_ok(d->out_stride_h, eo))
    return GQA_ERR_ALIGN;
  return GQA_OK;
}

// Split plan.  Chunk length T; n = ceil(max_seq / T) chunks.  The heuristic
// aims at ~768 workgroups (3 per compute unit) with at least one 32-key step
// per wave (T >= 128, a multiple of 128).
void decode_plan(const gqa_decode_desc* d, int32_t* T, int32_t* n) {
  int64_t t;
  if (d->kv_split_tokens >= d->max_seq) {
    t = d->max_seq;
  } else if (d->kv_split_tokens > 0) {
    t = d->kv_split_tokens;
  } else {
    const int64_t base = (int64_t)d->batch * d->num_kv_heads;
    const int64_t want = (768 + base - 1) / base;
    t = ((int64_t)d->max_seq + want - 1) / want;
    t = ((t + 127) / 128) * 128;
    if (t < 128) t = 128;
    if (t > d->max_seq) t = d->max_seq;
  }
  if (d->block_size != 0 && t < d->max_seq) t = (t + 31) / 32 * 32;   // paged: steps never straddle pages
  if (t > d->max_seq) t = d->max_seq;
  *T = (int32_t)t;
  *n = (int32_t)(((int64_t)d->max_seq + t - 1) / t);
}

// Chunks per partition workgroup.  With few (b, KV head) groups and many
// chunks, each workgroup streams several consecutive chunks (one partial per
// chunk) so that the grid is about one workgroup per compute unit; at least
// 4 workgroups per group.  With many groups (batched, ragged lengths) one
// chunk per workgroup keeps the load balanced.
constexpr int64_t kTargetWorkgroups = 256;
constexpr int64_t kMaxGroupsMultiChunk = 64;

int32_t decode_chunks_per_workgroup(const gqa_decode_desc* d, int32_t T, int32_t n) {
  if (n <= 1 || T % 32 != 0) return 1;
  const int64_t groups = (int64_t)d->batch * d->num_kv_heads;
  if (groups > kMaxGroupsMultiChunk) return 1;
  int64_t cpw = (int64_t)n * groups / kTargetWorkgroups;
  if (cpw > n / 4) cpw = n / 4;
  return cpw < 1 ? 1 : (int32_t)cpw;
}

// Decode workspace, with w = ceil(n / cpw) partition workgroups per (b, KV
// head), each writing one partial per query head of its group:
// [partial O: B * Hq * w * 128 f32] [partial (m, l): B * Hq * w * 2 f32].
int32_t decode_workgroups_per_group(const gqa_decode_desc* d, int32_t T, int32_t n) {
  const int32_t cpw = decode_chunks_per_workgroup(d, T, n);
  return (n + cpw - 1) / cpw;
}

size_t decode_ws_bytes(const gqa_decode_desc* d, int32_t T, int32_t n) {
  if (n <= 1) return 0;
  const size_t slots = (size_t)d->batch * (size_t)d->num_q_heads * (size_t)decode_workgroups_per_group(d, T, n);
  return slots * (GQA_ATTN_HEAD_DIM + 2) * sizeof(float);
}

// Prefill workgroup blocking: HC query heads (the largest divisor of G that is
// at most 8) times BQ query tokens, with HC * BQ / 32 <= 10 waves of 32 rows.
void prefill_blocking(int G, int32_t* HC, int32_t* BQ) {
  int hc = 1;
  for (int c = 1; c <= 8 && c <= G; ++c)
    if (G % c == 0) hc = c;
  int tb = gqa::kPrefillMaxWaves / hc;   // 32-token blocks per head
  if (tb > 4) tb = 4;
  if (tb < 1) tb = 1;
  *HC = hc;
  *BQ = 32 * tb;
}

gqa_status check_prefill_desc(const gqa_prefill_desc* d) {
  if (d == nullptr) return GQA_ERR_NULL;
  if (d->batch < 1 || d->num_q_heads < 1 || d->num_kv_heads < 1 || d->max_seq < 1) return GQA_ERR_SHAPE;
  if ((int64_t)d->batch * d->num_q_heads * ((d->max_seq + 31) / 32) > INT32_MAX) return GQA_ERR_SHAPE;
  if (d->num_q_heads % d->num_kv_heads != 0) return GQA_ERR_SHAPE;
  if (d->head_dim != GQA_ATTN_HEAD_DIM) return GQA_ERR_UNSUPPORTED;
  if (d->in_dtype != GQA_BF16 || !dtype_ok(d->out_dtype)) return GQA_ERR_UNSUPPORTED;
  if (d->causal != 0 && d->causal != 1) return GQA_ERR_SHAPE;
  if (d->write_k_cache != 0 && d->write_k_cache != 1) return GQA_ERR_SHAPE;
  if (d->block_size != 0) {   // paged: a power of two >= 16 rows per page, whole pages
    if (d->block_size < 16 || (d->block_size & (d->block_size - 1)) != 0 || d->max_seq % d->block_size != 0)
      return GQA_ERR_SHAPE;
  }
  // prefill addresses one (b, KV head) K / V slab with 32-bit byte offsets
  if ((int64_t)d->max_seq * d->k_stride_s * 2 + 512 > ((int64_t)1 << 32) ||
      (int64_t)d->max_seq * d->v_stride_s * 2 + 512 > ((int64_t)1 << 32))
    return GQA_ERR_UNSUPPORTED;
  const int ei = 2, eo = elem_size(d->out_dtype);
  const int64_t s[] = {d->q_stride_b, d->q_stride_h, d->q_stride_s, d->k_stride_b, d->k_stride_h, d->k_stride_s,
                       d->v_stride_b, d->v_stride_h, d->v_stride_s};
  for (int64_t x : s) {
    if (x < 0) return GQA_ERR_SHAPE;
  }
  if (d->out_stride_b < 0 || d->out_stride_h < 0 || d->out_stride_s < 0) return GQA_ERR_SHAPE;
  for (int64_t x : s) {
    if (!stride_ok(x, ei)) return GQA_ERR_ALIGN;
  }
  if (!stride_ok(d->out_stride_b, eo) || !stride_ok(d->out_stride_h, eo) || !stride_ok(d->out_stride_s, eo))
    return GQA_ERR_ALIGN;
  return GQA_OK;
}

}  // namespace

extern "C" {

const char* gqa_attn_status_string(gqa_status status) {
  switch (status) {
    case GQA_OK: return "GQA_OK";
    case GQA_ERR_NULL: return "GQA_ERR_NULL: a required pointer is NULL";
    case GQA_ERR_SHAPE: return "GQA_ERR_SHAPE: invalid size, head ratio or stride";
    case GQA_ERR_UNSUPPORTED: return "GQA_ERR_UNSUPPORTED: unsupported head_dim, dtype or group size";
    case GQA_ERR_ALIGN: return "GQA_ERR_ALIGN: pointer or stride not 16-byte aligned";
    case GQA_ERR_WORKSPACE: return "GQA_ERR_WORKSPACE: workspace missing or too small";
    case GQA_ERR_HIP: return "GQA_ERR_HIP: kernel launch failed";
    case GQA_ERR_SCRATCH: return "GQA_ERR_SCRATCH: the call needs more than the library's static decode scratch";
  }
  return "GQA_ERR_UNKNOWN: unknown status code";
}

int32_t gqa_attn_version(void) { return GQA_ATTN_VERSION; }

gqa_status gqa_attn_decode_plan(const gqa_decode_desc* desc, int32_t* split_tokens, int32_t* num_splits) {
  if (split_tokens == nullptr || num_splits == nullptr) return GQA_ERR_NULL;
  const gqa_status st = check_decode_desc(desc);
  if (st != GQA_OK) return st;
  decode_plan(desc, split_tokens, num_splits);
  return GQA_OK;
}

gqa_status gqa_attn_decode_workspace_size(const gqa_decode_desc* desc, size_t* bytes) {
  if (bytes == nullptr) return GQA_ERR_NULL;
  const gqa_status st = check_decode_desc(desc);
  if (st != GQA_OK) return st;
  int32_t T, n;
  decode_plan(desc, &T, &n);
  *bytes = decode_ws_bytes(desc, T, n);
  return GQA_OK;
}

}  // extern "C"

namespace {

// Validation shared by the decode entry points; fills the kernel parameters.
// need_inputs: q / caches / positions are used (partition); the merge needs
// only seq_lens, out and the workspace.
gqa_status prepare_decode(const gqa_decode_desc* d, const void* q, const void* k_cache, const void* v_cache,
                          const int32_t* seq_lens, const int32_t* positions, const void* q_norm_w,
                          const void* k_norm_w, float rope_theta, void* out, void* workspace,
                          size_t workspace_bytes, bool need_inputs, gqa::DecodeParams* p,
                          const int32_t* block_table = nullptr) {
  const gqa_status st = check_decode_desc(d);
  if (st != GQA_OK) return st;
  // a paged descriptor (block_size > 0) goes with gqa_attn_decode_paged only
  if (need_inputs && (d->block_size != 0) != (block_table != nullptr)) return GQA_ERR_SHAPE;
  if ((uintptr_t)block_table & 3u) return GQA_ERR_ALIGN;
  if (seq_lens == nullptr || out == nullptr) return GQA_ERR_NULL;
  if (need_inputs && (q == nullptr || k_cache == nullptr || v_cache == nullptr || positions == nullptr))
    return GQA_ERR_NULL;
  if (!aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache) || !aligned16(out) || !aligned16(q_norm_w) ||
      !aligned16(k_norm_w) || ((uintptr_t)seq_lens & 3u) || ((uintptr_t)positions & 3u))
    return GQA_ERR_ALIGN;
  int32_t T, n;
  decode_plan(d, &T, &n);
  const int64_t wgs = (int64_t)n * d->batch * d->num_kv_heads;
  if (wgs > INT32_MAX) return GQA_ERR_SHAPE;
  const size_t need = decode_ws_bytes(d, T, n);
  if (need > 0) {
    if (workspace == nullptr || workspace_bytes < need) return GQA_ERR_WORKSPACE;
    if (((uintptr_t)workspace & 255u) != 0) return GQA_ERR_ALIGN;
  }
  *p = gqa::DecodeParams{};
  p->q = q;
  p->k = k_cache;
  p->v = v_cache;
  p->seq_lens = seq_lens;
  p->positions = positions;
  p->q_norm_w = q_norm_w;
  p->k_norm_w = k_norm_w;
  p->out = out;
  const int32_t wpg = decode_workgroups_per_group(d, T, n);
  if (need > 0) {
    p->ws_o = (float*)workspace;
    p->ws_ml = p->ws_o + (size_t)d->batch * d->num_q_heads * wpg * GQA_ATTN_HEAD_DIM;
  }
  p->q_sb = d->q_stride_b;
  p->q_sh = d->q_stride_h;
  p->k_sb = d->k_stride_b;
  p->k_sh = d->k_stride_h;
  p->k_ss = d->k_stride_s;
  p->v_sb = d->v_stride_b;
  p->v_sh = d->v_stride_h;
  p->v_ss = d->v_stride_s;
  p->o_sb = d->out_stride_b;
  p->o_sh = d->out_stride_h;
  p->batch = d->batch;
  p->num_q_heads = d->num_q_heads;
  p->num_kv_heads = d->num_kv_heads;
  p->group = d->num_q_heads / d->num_kv_heads;
  p->max_seq = d->max_seq;
  p->split = T;
  p->n_split = n;
  p->cpw = decode_chunks_per_workgroup(d, T, n);
  p->wpg = wpg;
  p->out_bf16 = d->out_dtype == GQA_BF16;
  p->write_new_k = d->write_new_k != 0;
  if (block_table != nullptr) {
    p->block_table = block_table;
    p->block_log2 = __builtin_ctz((unsigned)d->block_size);
    p->max_blocks = d->max_seq / d->block_size;
  }
  p->eps = d->eps;
  p->scale_log2 = resolve_scale_log2(d->scale);
  p->rope_theta = rope_theta > 0.f ? (double)rope_theta : 0.0;
  p->rope_log2_theta = rope_theta > 0.f ? log2((double)rope_theta) : 0.0;
  return GQA_OK;
}

}  // namespace

extern "C" {

gqa_status gqa_attn_decode_partition(const gqa_decode_desc* d, const void* q, const void* k_cache,
                                     const void* v_cache, const int32_t* seq_lens, const int32_t* positions,
                                     const void* q_norm_w, const void* k_norm_w, float rope_theta, void* out,
                                     void* workspace, size_t workspace_bytes, hipStream_t stream) {
  gqa::DecodeParams p;
  const gqa_status st = prepare_decode(d, q, k_cache, v_cache, seq_lens, positions, q_norm_w, k_norm_w, rope_theta,
                                       out, workspace, workspace_bytes, true, &p);
  if (st != GQA_OK) return st;
  return gqa::launch_decode_partition(p, d->in_dtype == GQA_BF16, stream) == hipSuccess ? GQA_OK : GQA_ERR_HIP;
}

gqa_status gqa_attn_decode_merge(const gqa_decode_desc* d, const int32_t* seq_lens, void* out, void* workspace,
                                 size_t workspace_bytes, hipStream_t stream) {
  gqa::DecodeParams p;
  const gqa_status st = prepare_decode(d, nullptr, nullptr, nullptr, seq_lens, nullptr, nullptr, nullptr, 0.f, out,
                                       workspace, workspace_bytes, false, &p);
  if (st != GQA_OK) return st;
  return gqa::launch_decode_merge(p, stream) == hipSuccess ? GQA_OK : GQA_ERR_HIP;
}

gqa_status gqa_attn_decode(const gqa_decode_desc* d, const void* q, const void* k_cache, const void* v_cache,
                           const int32_t* seq_lens, const int32_t* positions, const void* q_norm_w,
                           const void* k_norm_w, float rope_theta, void* out, void* workspace,
                           size_t workspace_bytes, hipStream_t stream) {
  gqa::DecodeParams p;
  const gqa_status st = prepare_decode(d, q, k_cache, v_cache, seq_lens, positions, q_norm_w, k_norm_w, rope_theta,
                                       out, workspace, workspace_bytes, true, &p);
  if (st != GQA_OK) return st;
  if (gqa::launch_decode_partition(p, d->in_dtype == GQA_BF16, stream) != hipSuccess) return GQA_ERR_HIP;
  return gqa::launch_decode_merge(p, stream) == hipSuccess ? GQA_OK : GQA_ERR_HIP;
}

}  // extern "C"

namespace {

// ---- decode partials without a caller workspace: a file-scope device array
//      of GQA_ATTN_STATIC_SCRATCH_BYTES.  Each device that runs the library
//      holds its own copy (until the process ends) at its own address, found
//      once per device with hipGetSymbolAddress while that device is current;
//      host code passes only that address to kernels, never the array's name.
static __device__ __align__(256) uint8_t scratch[GQA_ATTN_STATIC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex scratch_mutex;
void* scratch_ptr[kMaxDevices] = {};

// Address of this device's scratch array (the current device's).
gqa_status device_scratch(void** ptr) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return GQA_ERR_HIP;
  if (dev < 0 || dev >= kMaxDevices) return GQA_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(scratch_mutex);
  if (scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) return GQA_ERR_HIP;
    scratch_ptr[dev] = p;
  }
  *ptr = scratch_ptr[dev];
  return GQA_OK;
}

}  // namespace

extern "C" {

gqa_status gqa_attn_decode_static(const gqa_decode_desc* d, const void* q, const void* k_cache, const void* v_cache,
                                  const int32_t* seq_lens, const int32_t* positions, const void* q_norm_w,
                                  const void* k_norm_w, float rope_theta, void* out, hipStream_t stream) {
  const gqa_status st = check_decode_desc(d);
  if (st != GQA_OK) return st;
  int32_t T, n;
  decode_plan(d, &T, &n);
  if (decode_ws_bytes(d, T, n) > GQA_ATTN_STATIC_SCRATCH_BYTES) return GQA_ERR_SCRATCH;
  // every argument check on the host first (a stand-in workspace address of
  // the right alignment and size), then the scratch address (HIP calls)
  gqa::DecodeParams p;
  gqa_status v = prepare_decode(d, q, k_cache, v_cache, seq_lens, positions, q_norm_w, k_norm_w, rope_theta, out,
                                (void*)(uintptr_t)256, GQA_ATTN_STATIC_SCRATCH_BYTES, true, &p);
  if (v != GQA_OK) return v;
  void* ws = nullptr;
  v = device_scratch(&ws);
  if (v != GQA_OK) return v;
  v = prepare_decode(d, q, k_cache, v_cache, seq_lens, positions, q_norm_w, k_norm_w, rope_theta, out, ws,
                     GQA_ATTN_STATIC_SCRATCH_BYTES, true, &p);
  if (v != GQA_OK) return v;
  if (gqa::launch_decode_partition(p, d->in_dtype == GQA_BF16, stream) != hipSuccess) return GQA_ERR_HIP;
  return gqa::launch_decode_merge(p, stream) == hipSuccess ? GQA_OK : GQA_ERR_HIP;
}

gqa_status gqa_attn_decode_paged(const gqa_decode_desc* d, const void* q, const void* k_pages, const void* v_pages,
                                 const int32_t* block_table, const int32_t* seq_lens, const int32_t* positions,
                                 const void* q_norm_w, const void* k_norm_w, float rope_theta, void* out,
                                 void* workspace, size_t workspace_bytes, hipStream_t stream) {
  if (d == nullptr) return GQA_ERR_NULL;
  if (d->block_size == 0) return GQA_ERR_SHAPE;
  if (block_table == nullptr) return GQA_ERR_NULL;
  gqa::DecodeParams p;
  const gqa_status st = prepare_decode(d, q, k_pages, v_pages, seq_lens, positions, q_norm_w, k_norm_w, rope_theta,
                                       out, workspace, workspace_bytes, true, &p, block_table);
  if (st != GQA_OK) return st;
  if (gqa::launch_decode_partition(p, d->in_dtype == GQA_BF16, stream) != hipSuccess) return GQA_ERR_HIP;
  return gqa::launch_decode_merge(p, stream) == hipSuccess ? GQA_OK : GQA_ERR_HIP;
}

gqa_status gqa_attn_prefill_workspace_size(const gqa_prefill_desc* desc, size_t* bytes) {
  if (bytes == nullptr) return GQA_ERR_NULL;
  const gqa_status st = check_prefill_desc(desc);
  if (st != GQA_OK) return st;
  *bytes = gqa::prefill_workspace_bytes(desc->batch, desc->num_q_heads, desc->num_kv_heads, desc->max_seq,
                                        desc->max_chunk > 0 ? desc->max_chunk : desc->max_seq, desc->causal != 0);
  return GQA_OK;
}

}  // extern "C"

namespace {

// Shared checks and parameters of gqa_attn_prefill and gqa_attn_prefill_chunk
// (past_lens != nullptr selects the chunked form).
gqa_status prepare_prefill(const gqa_prefill_desc* d, const void* q, const void* k, const void* v,
                           const int32_t* lens, const int32_t* past_lens, const int32_t* positions,
                           const void* q_norm_w, const void* k_norm_w, float rope_theta, void* out, void* workspace,
                           size_t workspace_bytes, gqa::PrefillParams* pp, const int32_t* block_table = nullptr) {
  gqa_status st = check_prefill_desc(d);
  if (st != GQA_OK) return st;
  // a paged descriptor (block_size > 0) goes with gqa_attn_prefill_chunk_paged only
  if ((d->block_size != 0) != (block_table != nullptr)) return GQA_ERR_SHAPE;
  if ((uintptr_t)block_table & 3u) return GQA_ERR_ALIGN;
  if (q == nullptr || k == nullptr || v == nullptr || lens == nullptr || positions == nullptr || out == nullptr)
    return GQA_ERR_NULL;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out) || !aligned16(q_norm_w) ||
      !aligned16(k_norm_w) || ((uintptr_t)lens & 3u) || ((uintptr_t)positions & 3u) || ((uintptr_t)past_lens & 3u))
    return GQA_ERR_ALIGN;
  if (d->write_k_cache && workspace == nullptr) return GQA_ERR_WORKSPACE;   // the write-back is phase 1's
  if (workspace != nullptr) {
    if (workspace_bytes < gqa::prefill_workspace_bytes(d->batch, d->num_q_heads, d->num_kv_heads, d->max_seq,
                                                       d->max_chunk > 0 ? d->max_chunk : d->max_seq, d->causal != 0))
      return GQA_ERR_WORKSPACE;
    if (((uintptr_t)workspace & 255u) != 0) return GQA_ERR_ALIGN;
  }
  gqa::PrefillParams& p = *pp;
  p = gqa::PrefillParams{};
  p.q = q;
  p.k = k;
  p.v = v;
  p.seq_lens = lens;
  p.past_lens = past_lens;
  if (block_table != nullptr) {
    p.block_table = block_table;
    p.block_log2 = __builtin_ctz((unsigned)d->block_size);
    p.max_blocks = d->max_seq / d->block_size;
  }
  p.positions = positions;
  p.q_norm_w = q_norm_w;
  p.k_norm_w = k_norm_w;
  p.out = out;
  p.q_sb = d->q_stride_b;
  p.q_sh = d->q_stride_h;
  p.q_ss = d->q_stride_s;
  p.k_sb = d->k_stride_b;
  p.k_sh = d->k_stride_h;
  p.k_ss = d->k_stride_s;
  p.v_sb = d->v_stride_b;
  p.v_sh = d->v_stride_h;
  p.v_ss = d->v_stride_s;
  p.o_sb = d->out_stride_b;
  p.o_sh = d->out_stride_h;
  p.o_ss = d->out_stride_s;
  p.batch = d->batch;
  p.num_q_heads = d->num_q_heads;
  p.num_kv_heads = d->num_kv_heads;
  p.group = d->num_q_heads / d->num_kv_heads;
  p.max_seq = d->max_seq;
  p.max_chunk = past_lens != nullptr && d->max_chunk > 0 ? d->max_chunk : d->max_seq;
  p.causal = d->causal;
  p.write_k_cache = d->write_k_cache;
  p.out_bf16 = d->out_dtype == GQA_BF16;
  prefill_blocking(p.group, &p.heads_per_wg, &p.block_q);
  p.n_qblocks = (d->max_seq + p.block_q - 1) / p.block_q;
  p.eps = d->eps;
  p.scale_log2 = resolve_scale_log2(d->scale);
  p.rope_theta = rope_theta > 0.f ? (double)rope_theta : 0.0;
  p.rope_log2_theta = rope_theta > 0.f ? log2((double)rope_theta) : 0.0;
  return GQA_OK;
}

}  // namespace

extern "C" {

gqa_status gqa_attn_prefill(const gqa_prefill_desc* d, const void* q, const void* k, const void* v,
                            const int32_t* seq_lens, const int32_t* positions, const void* q_norm_w,
                            const void* k_norm_w, float rope_theta, void* out, void* workspace,
                            size_t workspace_bytes, hipStream_t stream) {
  gqa::PrefillParams p;
  const gqa_status st = prepare_prefill(d, q, k, v, seq_lens, nullptr, positions, q_norm_w, k_norm_w, rope_theta,
                                        out, workspace, workspace_bytes, &p);
  if (st != GQA_OK) return st;
  const hipError_t e = workspace != nullptr ? gqa::launch_prefill_phased(p, workspace, stream)
                                            : gqa::launch_prefill_fused(p, stream);
  return e == hipSuccess ? GQA_OK : GQA_ERR_HIP;
}

// The two phases of gqa_attn_prefill with a workspace, as separate calls.
static gqa_status prefill_phase(const gqa_prefill_desc* d, const void* q, const void* k, const void* v,
                                const int32_t* seq_lens, const int32_t* positions, const void* q_norm_w,
                                const void* k_norm_w, float rope_theta, void* out, void* workspace,
                                size_t workspace_bytes, hipStream_t stream, int phase) {
  if (workspace == nullptr) return GQA_ERR_WORKSPACE;
  gqa::PrefillParams p;
  const gqa_status st = prepare_prefill(d, q, k, v, seq_lens, nullptr, positions, q_norm_w, k_norm_w, rope_theta,
                                        out, workspace, workspace_bytes, &p);
  if (st != GQA_OK) return st;
  return gqa::launch_prefill_phased(p, workspace, stream, phase) == hipSuccess ? GQA_OK : GQA_ERR_HIP;
}

gqa_status gqa_attn_prefill_keys(const gqa_prefill_desc* d, const void* q, const void* k, const void* v,
                                 const int32_t* seq_lens, const int32_t* positions, const void* q_norm_w,
                                 const void* k_norm_w, float rope_theta, void* out, void* workspace,
                                 size_t workspace_bytes, hipStream_t stream) {
  return prefill_phase(d, q, k, v, seq_lens, positions, q_norm_w, k_norm_w, rope_theta, out, workspace,
                       workspace_bytes, stream, gqa::kPhaseKeys);
}

gqa_status gqa_attn_prefill_attend(const gqa_prefill_desc* d, const void* q, const void* k, const void* v,
                                   const int32_t* seq_lens, const int32_t* positions, const void* q_norm_w,
                                   const void* k_norm_w, float rope_theta, void* out, void* workspace,
                                   size_t workspace_bytes, hipStream_t stream) {
  return prefill_phase(d, q, k, v, seq_lens, positions, q_norm_w, k_norm_w, rope_theta, out, workspace,
                       workspace_bytes, stream, gqa::kPhaseAttend);
}

gqa_status gqa_attn_prefill_chunk(const gqa_prefill_desc* d, const void* q, const void* k_cache,
                                  const void* v_cache, const int32_t* past_lens, const int32_t* chunk_lens,
                                  const int32_t* positions, const void* q_norm_w, const void* k_norm_w,
                                  float rope_theta, void* out, void* workspace, size_t workspace_bytes,
                                  hipStream_t stream) {
  if (d == nullptr) return GQA_ERR_NULL;
  if (d->max_chunk < 0) return GQA_ERR_SHAPE;
  const int64_t tmax = d->max_chunk > 0 ? d->max_chunk : d->max_seq;
  if ((int64_t)d->batch * d->num_q_heads * ((tmax + 31) / 32) > INT32_MAX) return GQA_ERR_SHAPE;
  if (past_lens == nullptr) return GQA_ERR_NULL;
  if (workspace == nullptr) return GQA_ERR_WORKSPACE;
  gqa::PrefillParams p;
  const gqa_status st = prepare_prefill(d, q, k_cache, v_cache, chunk_lens, past_lens, positions, q_norm_w, k_norm_w,
                                        rope_theta, out, workspace, workspace_bytes, &p);
  if (st != GQA_OK) return st;
  return gqa::launch_prefill_phased(p, workspace, stream) == hipSuccess ? GQA_OK : GQA_ERR_HIP;
}

gqa_status gqa_attn_prefill_chunk_paged(const gqa_prefill_desc* d, const void* q, const void* k_pages,
                                        const void* v_pages, const int32_t* block_table, const int32_t* past_lens,
                                        const int32_t* chunk_lens, const int32_t* positions, const void* q_norm_w,
                                        const void* k_norm_w, float rope_theta, void* out, void* workspace,
                                        size_t workspace_bytes, hipStream_t stream) {
  if (d == nullptr) return GQA_ERR_NULL;
  if (d->max_chunk < 0 || d->block_size == 0) return GQA_ERR_SHAPE;
  const int64_t tmax = d->max_chunk > 0 ? d->max_chunk : d->max_seq;
  if ((int64_t)d->batch * d->num_q_heads * ((tmax + 31) / 32) > INT32_MAX) return GQA_ERR_SHAPE;
  if (past_lens == nullptr || block_table == nullptr) return GQA_ERR_NULL;
  if (workspace == nullptr) return GQA_ERR_WORKSPACE;
  gqa::PrefillParams p;
  const gqa_status st = prepare_prefill(d, q, k_pages, v_pages, chunk_lens, past_lens, positions, q_norm_w,
                                        k_norm_w, rope_theta, out, workspace, workspace_bytes, &p, block_table);
  if (st != GQA_OK) return st;
  return gqa::launch_prefill_phased(p, workspace, stream) == hipSuccess ? GQA_OK : GQA_ERR_HIP;
}

}  // extern "C"
