/*
 * gqa_attn.h -- C ABI of the grouped-query fused attention library for
 * AMD Instinct MI355X (gfx950).
 *
 * The operation is the fused attention stage of a grouped-query-attention
 * decoder layer: a per-head RMSNorm ("QK-norm") and a rotary position
 * embedding (RoPE) applied to the projected query and key rows, then
 * softmax(scale * Q K^T) V where G = Hq / Hkv query heads share one KV head.
 *
 * Sources (the pages this library is built from):
 *  - "Qwen3-14B Optimization" (pypto-lib case study), section 2.1 "Shape 4"
 *    and change #796: QK-norm and RoPE are folded into the fused attention
 *    stage; change #602: the G query heads of one (KV head, batch) are
 *    batched into one tile, RoPE rotates the lo/hi halves of the head dim.
 *  - "ADR-0060: AHBM GQA Fused Attention Kernel (Llama3-70B)": section 0.5.3
 *    (inputs, softmax_scale = 1/sqrt(d)), section 0.5.4 (only O is an
 *    output; S and P are never materialised), section 3 (online softmax),
 *    section 4 (log-sum-exp merge of split partials), section 5.2 (decode,
 *    G heads folded into the matrix M dimension, query head h reads KV head
 *    floor(h / G)), section 5.4 (causal classification in prefill).
 *
 * Conventions shared by every entry point
 *  - All tensor pointers are DEVICE pointers (HIP device memory of the
 *    current device); seq_lens / positions are device int32 arrays.
 *  - Strides are in ELEMENTS.  The head dimension is always contiguous
 *    (stride 1) and must equal 128.
 *  - Tensor base pointers must be 16-byte aligned and every stride must be a
 *    multiple of 16 bytes (8 bf16 or 4 f32 elements): kernels use 128-bit
 *    loads.
 *  - The caller owns every buffer.  The library allocates nothing per call,
 *    keeps no mutable global state (calls are reentrant and thread-safe),
 *    never writes q, v or the norm weights, writes `out` (and `workspace`),
 *    and writes the key cache only where a descriptor asks for it (decode
 *    write_new_k: the new key's own row; prefill write_k_cache: the rows of
 *    the new tokens).  Calls are asynchronous on `stream`; the library
 *    never synchronises the host.
 *  - Every argument check except GQA_ERR_HIP happens on the host before any
 *    HIP call, so a rejected call has no device side effects.  No exception
 *    and no abort crosses this ABI.
 *  - Device-resident seq_lens are not checked on the host: kernels clamp a
 *    length L to [0, max_seq]; L = 0 yields an all-zero output row.
 *  - The prologue, per row x of 128 elements at RoPE position p:
 *        y = x * (mean(x^2) + eps)^(-1/2) * gamma      (skipped if gamma NULL)
 *        (y_i, y_{i+64}) <- (y_i cos a - y_{i+64} sin a,
 *                            y_{i+64} cos a + y_i sin a),
 *        a = p * theta^(-2i/128), i in [0, 64)          (skipped if theta <= 0)
 *    gamma is one [128] vector shared by all heads, in `in_dtype`.
 *    Angles are formed and range-reduced in double precision.
 */
#ifndef GQA_ATTN_H
#define GQA_ATTN_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define GQA_ATTN_HEAD_DIM 128
#define GQA_ATTN_MAX_GROUP 16      /* largest supported G = Hq / Hkv in decode */
#define GQA_ATTN_VERSION 3
/* bytes of the device array that gqa_attn_decode_static keeps its partials in */
#define GQA_ATTN_STATIC_SCRATCH_BYTES (16u << 20)

typedef enum gqa_status {
  GQA_OK = 0,
  GQA_ERR_NULL = 1,        /* a required pointer is NULL                          */
  GQA_ERR_SHAPE = 2,       /* non-positive size, Hq % Hkv != 0, bad stride        */
  GQA_ERR_UNSUPPORTED = 3, /* head_dim != 128, dtype, G too large, prefill f32,
                              decode cache slab of one (b, head) >= 4 GiB        */
  GQA_ERR_ALIGN = 4,       /* base pointer or stride not 16-byte aligned          */
  GQA_ERR_WORKSPACE = 5,   /* workspace NULL or smaller than required             */
  GQA_ERR_HIP = 6,         /* a kernel launch failed (its hipLaunchKernel status) */
  GQA_ERR_SCRATCH = 7      /* gqa_attn_decode_static: partials exceed the static
                              scratch (GQA_ATTN_STATIC_SCRATCH_BYTES)             */
} gqa_status;

typedef enum gqa_dtype {
  GQA_F32 = 0,
  GQA_BF16 = 1
} gqa_dtype;

/* Decode: one new token per sequence (T_q = 1). */
typedef struct gqa_decode_desc {
  int32_t batch;           /* B >= 1                                               */
  int32_t num_q_heads;     /* Hq >= 1                                              */
  int32_t num_kv_heads;    /* Hkv >= 1, Hq % Hkv == 0, Hq / Hkv <= 16             */
  int32_t head_dim;        /* must be 128                                          */
  int32_t max_seq;         /* cache capacity: rows [0, max_seq) of each (b, head)  */
  int32_t in_dtype;        /* gqa_dtype of q, k_cache, v_cache, q_norm_w, k_norm_w */
  int32_t out_dtype;       /* gqa_dtype of out                                     */
  int32_t kv_split_tokens; /* keys per split-KV chunk: 0 = library heuristic,
                              >= max_seq = one chunk (no merge); any T >= 1 ok    */
  int64_t q_stride_b, q_stride_h;               /* q[b, h, :]                      */
  int64_t k_stride_b, k_stride_h, k_stride_s;   /* k_cache[b, h, s, :]             */
  int64_t v_stride_b, v_stride_h, v_stride_s;   /* v_cache[b, h, s, :]             */
  int64_t out_stride_b, out_stride_h;           /* out[b, h, :]                    */
  float eps;               /* RMSNorm epsilon (e.g. 1e-6)                          */
  float scale;             /* softmax scale; <= 0 selects 1/sqrt(head_dim)         */
  int32_t write_new_k;     /* 1: store K'_{L-1} into k_cache[b, kv, L-1] (below)   */
  int32_t block_size;      /* 0: contiguous caches; > 0: rows per page of a paged
                              cache (gqa_attn_decode_paged only), a power of two
                              >= 32 dividing max_seq                               */
} gqa_decode_desc;

/* Prefill: self-attention over seq_lens[b] tokens per sequence (T_q = S_kv). */
typedef struct gqa_prefill_desc {
  int32_t batch;           /* B >= 1                                               */
  int32_t num_q_heads;     /* Hq                                                   */
  int32_t num_kv_heads;    /* Hkv, Hq % Hkv == 0                                   */
  int32_t head_dim;        /* must be 128                                          */
  int32_t max_seq;         /* S: token rows per sequence in q / k / v / out        */
  int32_t in_dtype;        /* must be GQA_BF16 (products on fp16 MFMA, whose 11-bit
                              operands cannot carry f32 inputs to their 1e-5 bound) */
  int32_t out_dtype;       /* GQA_F32 or GQA_BF16                                  */
  int32_t causal;          /* 1: query i sees keys j <= i; 0: all keys < S_b       */
  int64_t q_stride_b, q_stride_h, q_stride_s;
  int64_t k_stride_b, k_stride_h, k_stride_s;
  int64_t v_stride_b, v_stride_h, v_stride_s;
  int64_t out_stride_b, out_stride_h, out_stride_s;
  float eps;
  float scale;             /* <= 0 selects 1/sqrt(head_dim)                        */
  int32_t max_chunk;       /* gqa_attn_prefill_chunk only: query / output rows per
                              sequence (T_max); 0 means max_seq                   */
  int32_t block_size;      /* 0: contiguous caches; > 0: rows per page of a paged
                              cache (gqa_attn_prefill_chunk_paged only), a power
                              of two >= 16 dividing max_seq                        */
  int32_t write_k_cache;   /* 1: each new token's key row receives its
                              post-prologue value (below); needs a workspace     */
} gqa_prefill_desc;

/* Human-readable name of a status code (static storage; never NULL). */
const char* gqa_attn_status_string(gqa_status status);

/* Version of this ABI (GQA_ATTN_VERSION). */
int32_t gqa_attn_version(void);

/*
 * Split plan for a decode call (host only, no HIP call): the chunk length T
 * the call will use and the number of chunks n = ceil(max_seq / T).  Chunk c
 * covers keys [c*T, min((c+1)*T, L)) of a sequence of length L
 * (ADR-0060 section 2.2 contiguous blocks; section 4 merge).
 */
gqa_status gqa_attn_decode_plan(const gqa_decode_desc* desc, int32_t* split_tokens, int32_t* num_splits);

/*
 * Bytes of device workspace gqa_attn_decode needs for `desc` (host only, no
 * HIP call).  0 when the plan has a single chunk.  The workspace holds one
 * unnormalised partial (m, l, O[128]) in f32 per (b, q head, partition
 * workgroup); a partition workgroup sweeps c >= 1 consecutive chunks (c > 1
 * only with few (b, KV head) groups and many chunks, to keep the grid near
 * one workgroup per compute unit), so there are ceil(n / c) per (b, q head).
 */
gqa_status gqa_attn_decode_workspace_size(const gqa_decode_desc* desc, size_t* bytes);

/*
 * Grouped-query decode attention with the fused QK-norm + RoPE prologue
 * ("Qwen3-14B Optimization" 2.1 / #796; ADR-0060 sections 3, 4, 5.2).
 *
 * For each sequence b with L = clamp(seq_lens[b], 0, max_seq) and each
 * query head h (KV head kv = floor(h / G)):
 *   q'   = prologue(q[b, h, :], q_norm_w, positions[b])
 *   K'_j = k_cache[b, kv, j, :]                         for j < L-1
 *          (already post-prologue: cached keys are never re-rotated)
 *   K'_{L-1} = prologue(k_cache[b, kv, L-1, :], k_norm_w, positions[b])
 *          (the raw projected key of the token being decoded)
 *   out[b, h, :] = sum_j softmax_j(scale * q' . K'_j) v_cache[b, kv, j, :]
 * Rows j >= L of the caches are never read.  With desc->write_new_k == 0 the
 * caches are not written.  With write_new_k == 1, k_cache[b, kv, L-1, :] is
 * overwritten with K'_{L-1} rounded to in_dtype once the call has read it
 * ("Qwen3-14B Optimization" Shape 4: the rope phase writes the rotated key
 * into the KV-cache slot), so that the cache holds post-prologue keys for the
 * next step; only the one workgroup whose chunk holds slot L-1 reads or
 * writes that row, after its own reads.  v_cache is never written (V has no
 * prologue; its row L-1 is already in place).  When the prologue is off (no
 * k_norm_w and rope_theta <= 0) K'_{L-1} is the raw row and nothing is
 * written.
 *
 * q: [B, Hq, 128] (strides q_stride_*); k_cache, v_cache: [B, Hkv, max_seq,
 * 128]; seq_lens, positions: [B] int32 (device); q_norm_w, k_norm_w: [128]
 * in in_dtype or NULL; rope_theta <= 0 disables RoPE; out: [B, Hq, 128] in
 * out_dtype.  workspace: device buffer of at least
 * gqa_attn_decode_workspace_size bytes, 256-byte aligned (may be NULL when
 * that size is 0); its contents on entry are ignored.  Calls that share a
 * workspace must not run concurrently.
 * Errors: GQA_ERR_NULL, GQA_ERR_SHAPE (also: more than 2^31 - 1 workgroups),
 * GQA_ERR_UNSUPPORTED, GQA_ERR_ALIGN, GQA_ERR_WORKSPACE (checked on the
 * host), GQA_ERR_HIP (launch failure).
 */
gqa_status gqa_attn_decode(const gqa_decode_desc* desc, const void* q, const void* k_cache,
                           const void* v_cache, const int32_t* seq_lens, const int32_t* positions,
                           const void* q_norm_w, const void* k_norm_w, float rope_theta, void* out,
                           void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * The two steps of gqa_attn_decode as separate calls (same descriptor, same
 * plan, same workspace).  gqa_attn_decode(...) is exactly
 * gqa_attn_decode_partition(...) followed by gqa_attn_decode_merge(...) on
 * the same stream.
 *
 * gqa_attn_decode_partition: the split-KV partition step (ADR-0060 sections
 * 3 and 5.2 with the fused prologue).  Each partition workgroup (b, KV head,
 * a run of c consecutive chunks) writes one unnormalised partial (m, l, O)
 * per query head of its group to `workspace`: the log-sum-exp merge of its
 * chunks' partials (m in log2 units: scores are scaled by log2(e)).  When the
 * plan has a single chunk it writes the normalised result to `out` instead
 * and needs no workspace.
 *
 * gqa_attn_decode_merge: the log-sum-exp merge step (ADR-0060 section 4):
 * out[b, h, :] = sum_w 2^(m_w - M) O_w / sum_w 2^(m_w - M) l_w over the
 * ceil(L / (c T)) partition workgroups that hold keys; L = 0 writes zeros.  Reads only
 * `workspace` and seq_lens; a no-op returning GQA_OK when the plan has a
 * single chunk.
 * Errors: as gqa_attn_decode.
 */
gqa_status gqa_attn_decode_partition(const gqa_decode_desc* desc, const void* q, const void* k_cache,
                                     const void* v_cache, const int32_t* seq_lens, const int32_t* positions,
                                     const void* q_norm_w, const void* k_norm_w, float rope_theta, void* out,
                                     void* workspace, size_t workspace_bytes, hipStream_t stream);

gqa_status gqa_attn_decode_merge(const gqa_decode_desc* desc, const int32_t* seq_lens, void* out, void* workspace,
                                 size_t workspace_bytes, hipStream_t stream);

/*
 * gqa_attn_decode without a workspace argument, for callers that cannot
 * allocate device memory: code under HIP graph capture, serving loops and
 * harnesses that forbid allocation.  Same computation, outputs, plan and
 * kernels as gqa_attn_decode (bitwise the same out), with the split-KV
 * partials kept in a file-scope device array of GQA_ATTN_STATIC_SCRATCH_BYTES
 * (16 MiB) that every device running the library holds until the process
 * ends.  The call allocates nothing (no hipMalloc, no allocating library
 * routine); its first call on a device looks up that device's copy of the
 * array (hipGetSymbolAddress, with the device current) and keeps the address.
 * Every call on one device shares its array: calls that overlap on a device
 * (other streams, other host threads) race and must be serialised by the
 * caller; the array's contents between calls are unspecified (nothing in it
 * needs to start at zero).  Plans needing at most the array's bytes are
 * accepted (gqa_attn_decode_workspace_size reports what a descriptor needs).
 * Errors: as gqa_attn_decode (no GQA_ERR_WORKSPACE); GQA_ERR_SCRATCH when the
 * plan needs more than the array holds (checked on the host before any HIP
 * call); GQA_ERR_HIP also when the array's address cannot be looked up.
 */
gqa_status gqa_attn_decode_static(const gqa_decode_desc* desc, const void* q, const void* k_cache,
                                  const void* v_cache, const int32_t* seq_lens, const int32_t* positions,
                                  const void* q_norm_w, const void* k_norm_w, float rope_theta, void* out,
                                  hipStream_t stream);

/*
 * Decode over a paged KV cache (block table; the layout a serving engine's
 * fused attention consumes).  Same computation and outputs as gqa_attn_decode
 * (including write_new_k), with logical cache row j of sequence b at
 *   k_pages[block_table[b * (max_seq / bs) + j / bs], kv, j % bs, :]
 * (bs = desc->block_size; likewise v_pages), where the element strides are
 * k_stride_b = between pages, k_stride_h = between heads inside a page,
 * k_stride_s = between rows (same for v).  block_table: [B][max_seq / bs]
 * int32 page indices (device); entries for blocks at or past
 * ceil(seq_lens[b] / bs) are not read.  The split-KV chunk length is rounded
 * up to a multiple of 32 keys, so no 32-key step crosses a page.
 * Errors: as gqa_attn_decode; GQA_ERR_NULL for a missing block_table,
 * GQA_ERR_SHAPE for block_size == 0 here, or != 0 with the contiguous entry
 * points, or not a power of two >= 32 dividing max_seq.
 */
gqa_status gqa_attn_decode_paged(const gqa_decode_desc* desc, const void* q, const void* k_pages,
                                 const void* v_pages, const int32_t* block_table, const int32_t* seq_lens,
                                 const int32_t* positions, const void* q_norm_w, const void* k_norm_w,
                                 float rope_theta, void* out, void* workspace, size_t workspace_bytes,
                                 hipStream_t stream);

/*
 * Bytes of the optional prefill workspace (host only, no HIP call), for
 * gqa_attn_prefill and the chunked forms alike:
 * B * Hkv * ceil(max_seq / 32) * 9216 * 2 for the key tiles (per 32-key
 * tile, the K' rows (norm + RoPE applied) and the V rows, both in fp16, in
 * the padded row layout the attention tiles have in on-chip memory), plus,
 * when the attention grid would have fewer than 384 workgroups (B * Hq *
 * ceil(T_max / 128)), room to split long key ranges over several
 * workgroups: one counter per (b, q head, 128-query block) and one partial
 * (m, l, O) of 66 KiB per (b, q head, 128-query block, key span), with at
 * most 16 spans of at least 32 key tiles each.
 */
gqa_status gqa_attn_prefill_workspace_size(const gqa_prefill_desc* desc, size_t* bytes);

/*
 * Grouped-query causal prefill attention with the fused QK-norm + RoPE
 * prologue (ADR-0060 sections 3 and 5.4; "Qwen3-14B Optimization" 2.1).
 *
 * For each sequence b with n = clamp(seq_lens[b], 0, max_seq), every token
 * s < n sits at RoPE position positions[b] + s; both its query row (every
 * head) and its key row go through the prologue.  Query i of head h attends
 * keys j <= i (causal) or j < n (non-causal) of KV head floor(h / G):
 *   out[b, h, i, :] = sum_j softmax_j(scale * q'_i . k'_j) v[b, kv, j, :]
 * Rows s >= n of out are not written; rows s >= n of q / k / v are not read.
 *
 * q: [B, Hq, max_seq, 128]; k, v: [B, Hkv, max_seq, 128]; out: [B, Hq,
 * max_seq, 128].  in_dtype must be GQA_BF16.  QK^T and P V run on fp16 MFMA
 * with f32 accumulation: q', k' and P are rounded to fp16 (round to nearest
 * even) and v converted to fp16 before the products.  The conversion of a
 * bf16 input is exact for magnitudes in [2^-14, 65504] and loses at most
 * 2^-25 absolute below.  Beyond that range the conversion saturates: an
 * element of v or k' (after the prologue), or of q' (the two-phase path
 * carries the softmax scale times log2(e) in q', so there the bound applies
 * to q' * scale * log2(e)), whose magnitude exceeds 65504 enters the products
 * as +-65504, and the result is that of the inputs so clamped (finite; NaN
 * inputs stay NaN).  With the RMSNorm on, |q'|, |k'| are at most
 * sqrt(128) max|gamma|.
 *
 * workspace: optional.  With a device buffer of at least
 * gqa_attn_prefill_workspace_size bytes (256-byte aligned; contents on entry
 * ignored) the call runs in two phases on `stream`, the GPU form of the fused
 * stage's rope phase and attention phase separated by a grid-wide barrier:
 * every key row's prologue is computed once into the workspace, then the
 * attention kernel applies the query prologue as it loads query tiles.  With
 * workspace == NULL a single kernel recomputes the key prologue for every
 * (query block, key tile) pair (no workspace, more arithmetic).  Calls that
 * share a workspace must not run concurrently (the key tiles, and the split
 * counters the call resets, are per call).
 *
 * desc->write_k_cache == 1 (two-phase path only) makes the key phase store,
 * for every token s < n, k'_s rounded to bf16 over k[b, kv, s, :] after it has
 * read that row ("Qwen3-14B Optimization" 2.1 Shape 4: the rope phase writes
 * the rotated key into its KV-cache slot), so that k then holds the
 * post-prologue keys a later chunked prefill or decode reads as its cache.
 * Each row is read and written by the same threads and read by nothing else
 * in the call; the attention phase reads only the workspace.  v is never
 * written.  With the prologue off (no k_norm_w and rope_theta <= 0) nothing
 * is written.
 * Errors: as gqa_attn_decode; GQA_ERR_WORKSPACE for write_k_cache without a
 * workspace; GQA_ERR_SHAPE for write_k_cache not 0 or 1.
 */
gqa_status gqa_attn_prefill(const gqa_prefill_desc* desc, const void* q, const void* k, const void* v,
                            const int32_t* seq_lens, const int32_t* positions, const void* q_norm_w,
                            const void* k_norm_w, float rope_theta, void* out, void* workspace,
                            size_t workspace_bytes, hipStream_t stream);

/*
 * The two phases of gqa_attn_prefill with a workspace, as separate calls with
 * the same arguments (workspace required).  gqa_attn_prefill(..., workspace,
 * ...) is exactly gqa_attn_prefill_keys(...) followed by
 * gqa_attn_prefill_attend(...) on the same stream.
 *
 * gqa_attn_prefill_keys: the key prologue of every key row into the
 * workspace (and, with write_k_cache, into k); writes nothing to `out`.
 * gqa_attn_prefill_attend: attention of every query row (query prologue
 * applied on load) over the keys the workspace holds; reads q, v (through the
 * workspace), positions, seq_lens, q_norm_w and the workspace, writes `out`.
 * The workspace must hold the key phase of the same descriptor, inputs and
 * lengths; the attention phase may be repeated over it (its split counters
 * return to zero at the end of every call).
 * Errors: as gqa_attn_prefill; GQA_ERR_WORKSPACE for a missing workspace.
 */
gqa_status gqa_attn_prefill_keys(const gqa_prefill_desc* desc, const void* q, const void* k, const void* v,
                                 const int32_t* seq_lens, const int32_t* positions, const void* q_norm_w,
                                 const void* k_norm_w, float rope_theta, void* out, void* workspace,
                                 size_t workspace_bytes, hipStream_t stream);

gqa_status gqa_attn_prefill_attend(const gqa_prefill_desc* desc, const void* q, const void* k, const void* v,
                                   const int32_t* seq_lens, const int32_t* positions, const void* q_norm_w,
                                   const void* k_norm_w, float rope_theta, void* out, void* workspace,
                                   size_t workspace_bytes, hipStream_t stream);

/*
 * Chunked prefill ("ADR-0060: AHBM GQA Fused Attention Kernel (Llama3-70B)"
 * section 5.4: a query block of T_q tokens that may be a chunk of a longer
 * sequence; section 0.5.1 P2: cached keys are post-RoPE and never re-rotated).
 *
 * For sequence b, P = clamp(past_lens[b], 0, max_seq) tokens are already in
 * the cache and T = clamp(chunk_lens[b], 0, min(T_max, max_seq - P)) new
 * tokens follow (T_max = desc->max_chunk, or max_seq when 0).  Cache row j
 * sits at RoPE position positions[b] + j.  Rows j < P of k_cache hold
 * post-prologue keys; rows P <= j < P + T hold the raw projected keys of the
 * chunk, v_cache rows j < P + T the values.  Query t of the chunk (q[b, h, t],
 * raw) is token P + t: it goes through the prologue at position
 * positions[b] + P + t and attends keys j <= P + t (causal: the causal mask
 * is aligned at the bottom right of the T x (P + T) score matrix) or all
 * j < P + T (non-causal), of KV head floor(h / G):
 *   out[b, h, t, :] = sum_j softmax_j(scale * q'_t . K'_j) v_cache[b, kv, j, :]
 * Rows t >= T of out are not written; cache rows j >= P + T are not read.
 * With desc->write_k_cache == 1 the chunk's key rows P <= j < P + T receive
 * their post-prologue values (bf16), as in gqa_attn_prefill, so the cache
 * holds post-prologue keys for the next chunk or decode step; otherwise the
 * caches are not written.  With P = 0 this is gqa_attn_prefill over the chunk.
 *
 * q, out: [B, Hq, T_max, 128] (strides q_stride_* / out_stride_*); k_cache,
 * v_cache: [B, Hkv, max_seq, 128]; past_lens, chunk_lens, positions: [B]
 * int32 (device).  in_dtype must be GQA_BF16.  workspace is required
 * (gqa_attn_prefill_workspace_size bytes for the same descriptor, 256-byte
 * aligned, contents on entry ignored): the key prologue of the chunk rows
 * and the copy of the cached rows into the attention tile layout run first,
 * then the attention kernel.
 * Errors: as gqa_attn_prefill; GQA_ERR_NULL also for past_lens,
 * GQA_ERR_WORKSPACE for a missing workspace, GQA_ERR_SHAPE for max_chunk < 0.
 */
gqa_status gqa_attn_prefill_chunk(const gqa_prefill_desc* desc, const void* q, const void* k_cache,
                                  const void* v_cache, const int32_t* past_lens, const int32_t* chunk_lens,
                                  const int32_t* positions, const void* q_norm_w, const void* k_norm_w,
                                  float rope_theta, void* out, void* workspace, size_t workspace_bytes,
                                  hipStream_t stream);

/*
 * gqa_attn_prefill_chunk over a paged KV cache: cache row j of sequence b is
 *   k_pages[block_table[b * (max_seq / bs) + j / bs], kv, j % bs, :]
 * (bs = desc->block_size; likewise v_pages), with element strides k_stride_b =
 * between pages, k_stride_h = between heads inside a page, k_stride_s =
 * between rows.  block_table: [B][max_seq / bs] int32 page indices (device);
 * entries for blocks at or past ceil((past_lens[b] + T) / bs) are not read.
 * Everything else is as gqa_attn_prefill_chunk.
 * Errors: as gqa_attn_prefill_chunk; GQA_ERR_NULL for a missing block_table;
 * GQA_ERR_SHAPE for block_size == 0 here, or != 0 with the contiguous entry
 * points, or not a power of two >= 16 dividing max_seq.
 */
gqa_status gqa_attn_prefill_chunk_paged(const gqa_prefill_desc* desc, const void* q, const void* k_pages,
                                        const void* v_pages, const int32_t* block_table, const int32_t* past_lens,
                                        const int32_t* chunk_lens, const int32_t* positions, const void* q_norm_w,
                                        const void* k_norm_w, float rope_theta, void* out, void* workspace,
                                        size_t workspace_bytes, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* GQA_ATTN_H */
