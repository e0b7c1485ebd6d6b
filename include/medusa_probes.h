/*
 * medusa_probes.h -- device peak probes for the verify step's roofline.
 *
 * The verify step's kernels are judged against two ceilings: HBM read
 * bandwidth (the Medusa heads' weight stream, the KV prefix and the
 * verification logits are read once each) and dense bf16 matrix-core
 * throughput (the tree attention over long prefixes).  The published
 * MI355X figures are 8 TB/s and 2.5 PFLOP/s; these calls measure what the
 * device delivers to kernels of the same access pattern, so that a kernel's
 * fraction can be stated against both.  They compute nothing of the method.
 * Same conventions as medusa_verify.h (device pointers, caller-owned memory,
 * asynchronous on `stream`, status codes).
 */
#ifndef MEDUSA_PROBES_H
#define MEDUSA_PROBES_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Bytes of the device scratch `sink` that the probes write (one value per
 * thread, so that no load or product can be optimised away). */
size_t medusa_probe_sink_bytes(void);

/* One linear pass of 16-byte non-temporal loads over buf (device, 16-byte
 * aligned, bytes > 0 a multiple of 16): every byte read once; one workgroup
 * of four waves per CU streams its contiguous share with 8 loads in flight
 * per thread (whole 128-byte lines per load).  Time it with events; bytes /
 * time is the streaming read bandwidth. */
int medusa_probe_read(const void *buf, size_t bytes, void *sink, void *stream);

/* One read pass over buf, and per workgroup w (w < medusa_probe_read_workgroups())
 * its start and end in stamps[2w] and stamps[2w + 1] (device, uint32): the
 * low 32 bits of the device's constant-rate clock (medusa_probe_clock_mhz()
 * ticks per microsecond; 0 when the rate cannot be queried).  Workgroups
 * are dispatched round-robin over the XCDs, so workgroup w streams on XCD
 * w mod 8: the stamps give each XCD's streaming time for an equal share.
 * pattern 0: the linear pass of medusa_probe_read.  pattern 1: buf read as
 * rows of 8 KiB in tiles of 8 rows, the access pattern of the heads' weight
 * stream at d = 4096 (each load 8 rows x 128 B, whole lines, non-temporal;
 * bytes a multiple of 64 KiB).  MEDUSA_ERR_NULL when stamps is NULL,
 * MEDUSA_ERR_PARAM for another pattern, MEDUSA_ERR_SHAPE for a size that
 * does not fit it, otherwise as medusa_probe_read. */
int medusa_probe_read_timed(const void *buf, size_t bytes, void *sink, uint32_t *stamps,
                            int pattern, void *stream);
int medusa_probe_read_workgroups(void);
double medusa_probe_clock_mhz(void);

/* 256 workgroups of four waves (one per SIMD), each wave running eight
 * independent chains of `iters` v_mfma_f32_32x32x16_bf16 on register
 * operands (no memory traffic); medusa_probe_mfma_flops(iters) is the work
 * of one call.
 * MEDUSA_ERR_PARAM when iters < 1. */
int medusa_probe_mfma(int iters, void *sink, void *stream);
double medusa_probe_mfma_flops(int iters);

#ifdef __cplusplus
}
#endif

#endif /* MEDUSA_PROBES_H */
