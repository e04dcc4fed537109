/*
 * gqa_timeline.h -- C ABI of the timeline build of the attention library
 * (libgqa_attn_timeline.so: the same sources as libgqa_attn.so compiled with
 * -DGQA_TIMELINE; every entry point of gqa_attn.h behaves the same).  It is a
 * measurement build, not part of the attention computation: each workgroup
 * of the decode partition kernel and of the prefill attention kernel takes
 * s_memrealtime stamps at fixed points of its work, so that the time of a
 * step can be split into its parts ("ADR-0060: AHBM GQA Fused Attention
 * Kernel (Llama3-70B)" section 9 names the pipeline depth of the K/V stream
 * as the lever of a KV-load-bound decode; section 5.4 classifies the
 * prefill's (query block, key tile) pairs, which sets each block's tiles).
 * Stamps are kept in LDS and written out once per workgroup, in ticks of the
 * constant real-time counter (gqa_timeline_clock_khz).  A workgroup with
 * nothing to do writes nothing: its words keep what gqa_timeline_clear left
 * (0).
 *
 * Stamps of workgroup w (blockIdx.x < GQA_TIMELINE_BLOCKS) are the words
 * GQA_TIMELINE_SLOTS * w + i of the kernel's array.
 *
 * GQA_TIMELINE_DECODE, the decode partition kernel:
 *   0  entry (the prologue wave; streaming wave 0 in the 4-wave form)
 *   1  the sequence length and position are known
 *   2  streaming wave 0 has requested its first K/V step
 *   3  the prologue (q', RoPE table, the new key's score) is done
 *   4  streaming wave 0 starts its sweep (after the workgroup barrier)
 *   5  streaming wave 0 has finished its sweep and handed its state over
 *   6  the workgroup's partial (or, unsplit, its output rows) is stored
 *   7  unused (0)
 * GQA_TIMELINE_PREFILL, the prefill attention kernel (second phase):
 *   0  entry
 *   1  thread 0's q rows have landed
 *   2  the query prologue is done
 *   3  the first K'/V tiles have landed (after the workgroup barrier)
 *   4  the tile loop is done
 *   5  exit: output rows written, or the span's partial stored and its
 *      arrival counted (split blocks; the last span's exit follows its merge)
 *   6  the number of 32-key tiles of the workgroup's key range (a count)
 *   7  unused (0)
 *
 * Return values: 0 on success, 1 for a NULL pointer, an unknown kernel or a
 * size beyond the array, or the hipError_t of a failed copy (> 1).  The calls
 * synchronise with the device (plain hipMemcpyToSymbol / FromSymbol).
 */
#ifndef GQA_TIMELINE_H
#define GQA_TIMELINE_H

#include <stddef.h>
#include <stdint.h>

#define GQA_TIMELINE_SLOTS 8
#define GQA_TIMELINE_BLOCKS 4096
#define GQA_TIMELINE_DECODE 0
#define GQA_TIMELINE_PREFILL 1

#ifdef __cplusplus
extern "C" {
#endif

/* Zero the stamp arrays of both kernels. */
int32_t gqa_timeline_clear(void);

/* Copy the first `words` words of a kernel's stamp array to host memory. */
int32_t gqa_timeline_read(int32_t kernel, uint64_t* host, size_t words);

/* The real-time counter's frequency in kHz (hipDeviceAttributeWallClockRate
 * of the current device). */
int32_t gqa_timeline_clock_khz(int32_t* khz);

#ifdef __cplusplus
}
#endif

#endif /* GQA_TIMELINE_H */
