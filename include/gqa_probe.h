/*
 * gqa_probe.h -- C ABI of the measurement probes that sit beside the grouped-
 * query attention library (libgqa_probe.so, gfx950).  They are not part of
 * the attention computation: they measure what the GPU itself allows, so
 * that the attention kernels' rooflines can be read against the machine.
 *
 *  - gqa_probe_read: a plain streaming read of `bytes` bytes from HBM (the
 *    floor of any kernel that has to read that much: the decode partition
 *    reads its K/V rows once, "ADR-0060: AHBM GQA Fused Attention Kernel
 *    (Llama3-70B)" section 11, HBM bytes independent of the group size).
 *  - gqa_probe_copy: a plain device copy of `bytes` bytes (read + write), the
 *    calibration kernel of the HBM byte counters (its FETCH_SIZE and
 *    WRITE_SIZE per dispatch are known exactly).
 *  - gqa_probe_empty: one empty workgroup, the dispatch floor of one kernel
 *    node in a replayed HIP graph.
 *
 * All pointers are device pointers.  src / dst must be 16-byte aligned and
 * bytes a multiple of 16.  sink is one device uint32 that the read probe
 * writes only when its XOR of every loaded word equals a fixed constant
 * (which keeps the loads alive; callers ignore its value).  Calls are
 * asynchronous on `stream`.  Return value: 0 on success, 1 for a NULL or
 * misaligned argument (checked on the host, before any HIP call), or the
 * hipError_t of a failed launch (> 1).
 */
#ifndef GQA_PROBE_H
#define GQA_PROBE_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

int32_t gqa_probe_read(const void* src, size_t bytes, uint32_t* sink, hipStream_t stream);
int32_t gqa_probe_copy(const void* src, void* dst, size_t bytes, hipStream_t stream);
int32_t gqa_probe_empty(hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* GQA_PROBE_H */
