/*
 * lsq_probe — device-memory streaming probe of liblsq (gfx950).  C ABI.
 *
 * Not part of the decode step: a plain read, write or copy stream over one
 * device buffer, timed by the caller, that measures the rate a hand-written
 * kernel reaches on this part (and, lsq_probe_valu below, the VALU issue rate
 * of one instruction form).  It is the practical ceiling against which the
 * decode step's bandwidth is judged: the step reads and rewrites its packed
 * state every token ("Preserving Updates in Low-Bit Recurrent State
 * Quantization", abstract: high-precision states cost memory and bandwidth at
 * large batch sizes), so a read-then-write stream is its bound.
 *
 * Kernel: workgroups of 256 lanes; each lane moves `loads_per_lane` 16-byte
 * vectors per iteration (all loads of an iteration are issued before any is
 * used), consecutive lanes take consecutive 16-byte vectors, and the grid
 * strides over the buffer.  kind READ sums the data into a value that is
 * written to `dst` (4 bytes) only if it equals a constant the data cannot
 * produce by chance; WRITE fills dst with a pattern; COPY copies src to dst.
 */
#ifndef LSQ_PROBE_H
#define LSQ_PROBE_H

#include "lsq.h"

#ifdef __cplusplus
extern "C" {
#endif

typedef enum { LSQ_PROBE_READ = 0, LSQ_PROBE_WRITE = 1, LSQ_PROBE_COPY = 2 } lsq_probe_kind;

/* One streaming pass, asynchronous on `stream` (a hipStream_t as void*).
 *   kind            lsq_probe_kind
 *   src             device buffer of `bytes` bytes, read by READ and COPY
 *                   (may be NULL for WRITE)
 *   dst             device buffer of `bytes` bytes written by WRITE and COPY;
 *                   for READ at least 4 bytes (written only by the check
 *                   described above)
 *   bytes           a multiple of 16; 0 is a no-op
 *   loads_per_lane  1, 2, 4 or 8 16-byte vectors per lane per iteration
 *   nontemporal     0: default loads and stores; 1: loads and stores carry
 *                   the non-temporal hint
 *   workgroups      grid size (>= 1), or 0 for one workgroup per
 *                   256 * loads_per_lane * 16 bytes (a single pass, no
 *                   strided loop)
 * Pointers must be 16-byte aligned.  INVALID_ARG for a bad kind, size,
 * alignment, loads_per_lane or a null buffer the kind needs; HIP for a launch
 * failure.  The caller owns both buffers; nothing is allocated. */
lsq_status lsq_probe_stream(int32_t kind, const void* src, void* dst, size_t bytes,
                            int32_t loads_per_lane, int32_t nontemporal, int32_t workgroups,
                            void* stream);

/* Span mode: every wave owns span_kib KiB of consecutive bytes (wave w the
 * span starting at byte w * span_kib * 1024), reads it 1 KiB per step with two
 * steps in flight (16 bytes per lane, non-temporal loads if nontemporal = 1)
 * and writes each KiB, with one bit flipped, to the same offset of dst with
 * non-temporal stores; dst may equal src (in place).  This is the access
 * pattern of a decode step whose waves each carry one head's packed state.
 *   span_kib  1, 2, 4, 8, 10 or 16
 *   bytes     a multiple of span_kib * 1024 (the waves cover exactly bytes)
 * Both pointers 16-byte aligned and non-null.  INVALID_ARG otherwise; HIP for
 * a launch failure. */
lsq_status lsq_probe_span(const void* src, void* dst, size_t bytes, int32_t span_kib,
                          int32_t nontemporal, void* stream);

typedef enum {
  LSQ_PROBE_VALU_FMA = 0,      /* v_fma_f32, every operand a VGPR */
  LSQ_PROBE_VALU_MED3 = 1,     /* v_med3_f32 */
  LSQ_PROBE_VALU_MIXED = 2,    /* four of each per iteration */
  /* one instruction each, written out in inline asm, every operand a VGPR: */
  LSQ_PROBE_VALU_FMAC = 3,     /* v_fmac_f32, the accumulating two-operand fma */
  LSQ_PROBE_VALU_FMA_MIX = 4,  /* v_fma_mix_f32 (a binary16 operand) */
  LSQ_PROBE_VALU_LSHL_OR = 5,  /* v_lshl_or_b32 */
  LSQ_PROBE_VALU_PERM = 6,     /* v_perm_b32 */
  LSQ_PROBE_VALU_XAD = 7,      /* v_xad_u32 */
  LSQ_PROBE_VALU_AND = 8,      /* v_and_b32 */
  LSQ_PROBE_VALU_MUL = 9       /* v_mul_f32 */
} lsq_probe_valu_form;

/* VALU issue probe: the rate at which this part retires one instruction form
 * when nothing else limits it, the reference for a kernel whose arithmetic,
 * not its memory traffic, sets its time (the packed-state decode step under
 * directional rounding is one).  `workgroups` workgroups of 256 lanes (4
 * waves); every lane runs `iters` iterations of eight independent chains of
 * the form, so one launch issues workgroups * 4 * iters * 8 wave64
 * instructions of it (1024 workgroups fill the chip's SIMDs four waves deep).
 * The rates of the forms price a kernel's instruction mix.  No memory is
 * read; out (4 bytes) is written only if the chains' sum equals a value they
 * cannot produce (forms 0-2), which keeps the compiler from removing them
 * (forms 3-9 are kept by their volatile asm and never write out).
 *   form        lsq_probe_valu_form
 *   workgroups  >= 1
 *   iters       >= 1
 * INVALID_ARG for a bad form or count or a null out; HIP for a launch
 * failure. */
lsq_status lsq_probe_valu(int32_t form, int32_t workgroups, int32_t iters, float* out,
                          void* stream);

#ifdef __cplusplus
}
#endif
#endif /* LSQ_PROBE_H */
