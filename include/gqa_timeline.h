/*
 * gqa_timeline.h -- C ABI of the timeline build of the attention library
 * (libgqa_attn_timeline.so: the same sources as libgqa_attn.so compiled with
 * -DGQA_TIMELINE; every entry point of gqa_attn.h behaves the same).  It is a
 * measurement build, not part of the attention computation: each workgroup
 * of the decode partition kernel takes s_memrealtime stamps at fixed points
 * of its work ("ADR-0060: AHBM GQA Fused Attention Kernel (Llama3-70B)"
 * section 9 names the pipeline depth of the K/V stream as the lever of a
 * KV-load-bound decode; the stamps show where a short step's time goes).
 *
 * Stamps of workgroup w (blockIdx.x < GQA_TIMELINE_BLOCKS) are the words
 * GQA_TIMELINE_SLOTS * w + i of the device array, in ticks of the constant
 * real-time counter (gqa_timeline_clock_khz):
 *   0  entry (the prologue wave; streaming wave 0 in the 4-wave form)
 *   1  the sequence length and position are known
 *   2  streaming wave 0 has requested its first K/V step
 *   3  the prologue (q', RoPE table, the new key's score) is done
 *   4  streaming wave 0 starts its sweep (after the workgroup barrier)
 *   5  streaming wave 0 has finished its sweep and handed its state over
 *   6  the workgroup's partial (or, unsplit, its output rows) is stored
 *   7  unused (0)
 * A workgroup that returns early (a range past the sequence) writes nothing:
 * its words keep what gqa_timeline_clear left (0).  Stamps are kept in LDS and
 * written once at the workgroup's end.  Only the partition kernel stamps.
 *
 * Return values: 0 on success, 1 for a NULL pointer or a size beyond the
 * array, or the hipError_t of a failed copy (> 1).  The calls synchronise
 * with the device (plain hipMemcpyToSymbol / hipMemcpyFromSymbol).
 */
#ifndef GQA_TIMELINE_H
#define GQA_TIMELINE_H

#include <stddef.h>
#include <stdint.h>

#define GQA_TIMELINE_SLOTS 8
#define GQA_TIMELINE_BLOCKS 4096

#ifdef __cplusplus
extern "C" {
#endif

/* Zero the device array of stamps. */
int32_t gqa_timeline_clear(void);

/* Copy the first `words` words of the device array to host memory. */
int32_t gqa_timeline_read(uint64_t* host, size_t words);

/* The real-time counter's frequency in kHz (hipDeviceAttributeWallClockRate
 * of the current device). */
int32_t gqa_timeline_clock_khz(int32_t* khz);

#ifdef __cplusplus
}
#endif

#endif /* GQA_TIMELINE_H */
