/*
 * lsq — decode step of a linear recurrence whose matrix state is stored at low
 * bit-width, for AMD Instinct MI355X (gfx950).  C ABI.
 *
 * The operation (one decode step, for every batch*head independently):
 *
 *   S_t = S_{t-1} Lambda_t (I - delta beta_t k_t k_t^T) + beta_t v_t k_t^T
 *
 * is Eq. (1) of "LinQuant: Functional Invariances for Low-Precision Linear
 * Recurrences" (summary page, Theoretical Foundation), with scalar decay
 * Lambda_t = alpha_t I or diagonal decay diag(alpha_t), write gate beta_t > 0
 * and delta in {0,1} (Key structural choices).  S_t is Dv x Dk.  The step
 * emits o_t = S_t q_t, then requantises the state, as "When Dynamic Scaling
 * Fails" (abstract) describes: the state is rewritten and requantised at every
 * decode step with uniform group-wise INT4/INT8, the group scale being
 *   DYNAMIC    read from the new state itself (per-token absmax; project page,
 *              mechanism paragraph),
 *   PERSISTENT frozen once by calibration (the abstract's persistent arm),
 *   YOKED      read from an fp32 reference state advanced alongside (the
 *              project page's control arm: the same quantiser, with the scale
 *              no longer fed back from the quantised state),
 * and rounded either to nearest-even or by Bounded Directional Rounding
 * ("Preserving Updates in Low-Bit Recurrent State Quantization", abstract): an
 * element whose rounded value moved opposite to its update is rounded one
 * grid step toward the update, or with a deterministic golden-ratio Weyl
 * dither ("Low-Discrepancy Dither for Quantized Recurrent State Caches",
 * listing entry; the sequence below is this library's reading of it).
 *
 * Arithmetic contract (every step below is what the kernels compute):
 *   m_c   = fl(s_group(c) * alpha_c)            alpha_c = alpha for scalar decay
 *   S'_c  = fl(C_c * m_c)                       dequantise with the decay folded in
 *   u     = dot(S', k)                          only when delta = 1, else 0
 *   w     = fl(beta * fl(v_r - u))
 *   S_c   = fma(w, k_c, S'_c)
 *   o_r   = dot(S, q)                           read before requantisation
 *   s_new = DYNAMIC: fl(max|S_c| / qmax) per group; PERSISTENT: s;
 *           YOKED: fl(max|R_c| / qmax) with R advanced by the same update in fp32
 *   inv   = s_new == 0 ? 0 : fl(1 / s_new)
 *   c1    = clamp(round-half-even(S_c * inv exactly), -qmax, qmax)
 *   BDR:    sigma_c = sign(w) sign(k_c); if (c1 - S'_c * inv) * sigma_c < 0
 *           (exact), then c = clamp(c1 + sigma_c), else c = c1
 *   DITHER: c = clamp(floor(S_c * inv + u_i) exactly, -qmax, qmax) in place of
 *           c1, u_i = ((i * 0x9E3779B9) mod 2^32 >> 9) * 2^-23 (the Weyl
 *           sequence frac(i (sqrt(5)-1)/2) in fixed point, 23 bits), i =
 *           (t Dv Dk + r Dk + c) mod 2^32 with t the handle's step index
 *   BDR_A, BDR_B (sensitivity flags; frozen scale s, stored code C_old): the
 *           readings of "update" and "move" not taken by BDR.  A: sigma_c =
 *           sign(S_c - C_old s) (exact); B': sigma_c = sign(w) sign(k_c).  If
 *           (c1 - C_old) * sigma_c < 0 and s > 0 then c = c1 + sigma_c, else c1.
 *           On a frozen grid A never fires (it equals RNE).
 * with qmax = 2^(bits-1) - 1 (7 for INT4, 127 for INT8).  dot(a, b) is an
 * fp32 sum in one fixed order (the pages leave the order open; fixing it makes
 * every code, scale and output reproducible bit for bit): the columns are
 * taken in consecutive blocks of 32, inside a block the products accumulate by
 * a chain of fused multiply-adds from zero in column order, and the block sums
 * are added in adjacent pairs, level by level ((b0 + b1) + (b2 + b3) at Dk =
 * 128).  The unquantised mode (bits 32) keeps the same formulas with its own
 * summation order.
 *
 * Memory: every pointer below is a DEVICE pointer (row-major, 16-byte
 * aligned) unless stated.  The library never allocates device memory: the
 * caller allocates the state buffers (lsq_state_sizes gives their sizes) and
 * the inputs/outputs, and binds them to a handle.  The handle itself is a
 * small host object.
 *
 * Packed state layout (per handle, heads = batch*heads):
 *   codes  [heads][Dv][Dk*bits/8] bytes.  INT8: one two's-complement byte per
 *          element.  INT4: element c of a row in byte c/2, low nibble for even
 *          c, two's-complement nibble.  Codes lie in [-qmax, qmax]; the
 *          most negative code (-8, -128) is never produced and is not a
 *          valid input.
 *   scales [heads][Dv][Dk/group], one per contiguous group along Dk: fp32,
 *          or (scale_fmt) IEEE binary16 or bfloat16 bit patterns, 2 bytes;
 *          group = 0: [heads] fp32, one per head.
 *   ref    [heads][Dv][Dk] fp32, the yoked policy's reference state.
 *   f32    [heads][Dv][Dk] fp32, the state of the unquantised mode (bits 32).
 *   lrb    Low-Rank Bypass buffer (lrb_rank = r > 0), fp32: a [heads][r][Dv]
 *          followed by b [heads][2][r][Dk] (copy 1 used by diagonal decay).
 *
 * Low-Rank Bypass ("Preserving Updates in Low-Bit Recurrent State
 * Quantization", abstract: small updates collect in a low-rank buffer, and
 * the parts of it that have grown large enough enter the state from time to
 * time; rank, period and threshold are not given there).  This
 * library's reading: slot j holds a_j [Dv], b_j [Dk], B = sum_j a_j b_j^T;
 * at step t, n = t mod r slots are filled (the handle's step index t).  The
 * buffer decays with the state (scalar decay: a_j = fl(alpha a_j); diagonal:
 * b_j = fl(b_j alpha)); u and o are taken from S' + B (o also includes the
 * new write); the write fills slot n (a_n = w, b_n = k) instead of entering
 * the quantised state, which is requantised from S' alone; when n = r-1 the
 * step merges instead: X = S' then X = fma(a_j, b_j, X) for j = 0..n in slot
 * order, the scale policy and rounding applied to X (BDR's update sign is the
 * sign of U built the same way from 0), and the buffer empties.  b is read from
 * copy t mod 2 and written to copy (t+1) mod 2 under diagonal decay (copy 0
 * only under scalar decay).  Supported: bits 4/8, DYNAMIC or PERSISTENT,
 * groups of 32 or more, r <= 8; the buffer starts as lsq_state_zero leaves it.
 * Inputs per step: q, k [heads][Dk]; v [heads][Dv]; alpha [heads] (scalar
 * decay) or [heads][Dk] (diagonal); beta [heads].  Output o [heads][Dv];
 * o_ref [heads][Dv] (yoked only, nullable).
 *
 * Errors and streams: calls are asynchronous on the given HIP stream (a
 * hipStream_t passed as void*, NULL for the default stream).  Argument checks
 * happen on the host before any launch and return a status without touching
 * the device.  Launch failures return LSQ_ERR_HIP.  No C++ exception crosses
 * the ABI.  A handle must not be used on two streams at once.  Inputs must be
 * finite and the state far from overflow (scales and |S| below 2^100); a
 * nonzero scale must be a normal float (>= 2^-126), since fl(1/s) overflows
 * below 2^-128 and 0 * inf has no code; the data is not scanned.  With batch*heads == 0 every call is a no-op and its
 * data pointers may be NULL.
 */
#ifndef LSQ_H
#define LSQ_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  LSQ_OK = 0,
  LSQ_ERR_INVALID_ARG = 1,     /* null pointer, bad value, misaligned buffer */
  LSQ_ERR_UNSUPPORTED = 2,     /* a valid configuration this library has no kernel for */
  LSQ_ERR_BUFFER_TOO_SMALL = 3,
  LSQ_ERR_NOT_CALIBRATED = 4,  /* persistent policy stepped before its scales were frozen */
  LSQ_ERR_HIP = 5              /* a HIP runtime call or kernel launch failed */
} lsq_status;

typedef enum {
  LSQ_POLICY_NONE = 0,        /* bits == 32: unquantised fp32 state */
  LSQ_POLICY_DYNAMIC = 1,
  LSQ_POLICY_PERSISTENT = 2,
  LSQ_POLICY_YOKED = 3
} lsq_policy;

/* BDR_A and BDR_B are the two readings of directional rounding this library
 * does not take, for sensitivity runs (persistent scale only, groups of 32 or
 * more, fp32 scales, no bypass; see the rounding contract above). */
typedef enum {
  LSQ_ROUND_RNE = 0,
  LSQ_ROUND_BDR = 1,
  LSQ_ROUND_DITHER = 2,
  LSQ_ROUND_BDR_A = 3,
  LSQ_ROUND_BDR_B = 4
} lsq_rounding;
typedef enum { LSQ_DECAY_SCALAR = 0, LSQ_DECAY_DIAG = 1 } lsq_decay;
typedef enum { LSQ_SCALE_F32 = 0, LSQ_SCALE_F16 = 1, LSQ_SCALE_BF16 = 2 } lsq_scale_format;

/* Shape, format and method flags of one handle.
 *   bits   4, 8 (quantised) or 32 (fp32 state, policy NONE)
 *   group  group size along Dk; must divide dk.  This library supports
 *          power-of-two groups of 16 to Dk elements (one lane owns 32
 *          consecutive elements of a row: one group, part of one, or two
 *          16-element groups) and Dk in {64, 128}.  group = Dk is one scale
 *          per row.  group = 0 is one scale per head for the whole Dv x Dk
 *          state (scales [heads] fp32): DYNAMIC (the absmax over every
 *          element after the step's update, so all rows are updated before
 *          any is requantised) or PERSISTENT (calibrated over the head), RNE
 *          or BDR, fp32 scale, no bypass, Dv <= 1024.  INT4 with 16-element
 *          groups and fp32 scales stores 6 bits per element, 5.33x less
 *          than an fp32 state.
 *   delta  0: linear write, 1: delta-rule correction
 *   scale_fmt  stored format of the group scales (the pages fix none; 16-bit
 *          scales are the scale-format variant of "Preserving Updates in
 *          Low-Bit Recurrent State Quantization", whose memory saving of at
 *          most 5.3x leaves the format open).  A computed scale (dynamic, yoked,
 *          calibration) is rounded to the format, to nearest with ties to
 *          even (binary16 with subnormals, overflow to infinity; bfloat16 on
 *          the upper half of the fp32 pattern), and the codes are formed with
 *          that stored value: inv = fl(1/s_stored); elements beyond qmax
 *          steps of a scale that rounded down clamp.  Quantised states only;
 *          not with the bypass.  INT4 g32 with bfloat16
 *          scales stores 4.5 bits per element (7.1x less than fp32), INT4
 *          g16 5 bits (6.4x).
 */
typedef struct {
  int32_t batch, heads, dk, dv;
  int32_t bits, group, policy, rounding, delta, decay;
  int32_t lrb_rank;   /* Low-Rank Bypass slots r, 0 (off) to 8; see below */
  int32_t scale_fmt;  /* lsq_scale_format (LSQ_SCALE_F32 = 0) */
} lsq_config;

/* Caller-owned device buffers and their capacities in bytes.  Buffers the
 * configuration does not use may be NULL with capacity 0. */
typedef struct {
  void* codes;   size_t codes_bytes;
  float* scales; size_t scales_bytes;
  float* ref;    size_t ref_bytes;
  float* f32;    size_t f32_bytes;
  float* lrb;    size_t lrb_bytes;    /* Low-Rank Bypass buffer (lrb_rank > 0) */
} lsq_buffers;

typedef struct lsq_state lsq_state;

/* Byte sizes of the state buffers a configuration needs (0 when unused).
 * Host only.  Any output pointer may be NULL. */
lsq_status lsq_state_sizes(const lsq_config* cfg, size_t* codes_bytes, size_t* scales_bytes,
                           size_t* ref_bytes, size_t* f32_bytes, size_t* lrb_bytes);

/* Create a handle that binds the caller's buffers.  Allocates only the host
 * handle.  Checks: valid config, non-null and 16-byte aligned buffers for
 * what the config uses, capacities >= lsq_state_sizes.  The buffer contents
 * are not read.  A persistent-policy handle starts uncalibrated. */
lsq_status lsq_state_alloc(const lsq_config* cfg, const lsq_buffers* bufs, lsq_state** out);

/* Destroy a handle (the device buffers stay the caller's).  NULL is a no-op. */
void lsq_state_free(lsq_state* st);

/* Copy of the handle's configuration (host). */
lsq_status lsq_state_config(const lsq_state* st, lsq_config* out);

/* S_0 = 0: zero codes, scales, ref and f32 with a fill kernel (capturable in
 * a HIP graph).  A persistent-policy handle becomes uncalibrated. */
lsq_status lsq_state_zero(lsq_state* st, void* stream);

/* Load an fp32 state S [heads][Dv][Dk] (device) into the handle: one scale per
 * group s = fl(absmax/qmax), codes clamp(RNE(S * fl(1/s))); the yoked policy
 * also copies S into ref; bits 32 copies S into f32.  Freezes the scales of a
 * persistent-policy handle (marks it calibrated).  This is the calibration of
 * the persistent-scale arm of "When Dynamic Scaling Fails" (abstract). */
lsq_status lsq_state_calibrate(lsq_state* st, const float* S, void* stream);

/* The dequantised state: S [heads][Dv][Dk] fp32 (device, caller-owned, 16-byte
 * aligned) receives fl(C s) for every element, C the stored code and s its
 * group's scale in the stored format (or the head's scale for group 0), the
 * value a step starts from before its decay ("Preserving Updates in Low-Bit
 * Recurrent State Quantization", abstract: the low-bit state stands for the
 * full-precision one; its norm against an fp32 reference is the quantity of
 * "When Dynamic Scaling Fails", norm-inflation figure).  bits 32 copies the
 * fp32 state.  Asynchronous on stream; the handle is not changed.
 * INVALID_ARG for a null or misaligned S. */
lsq_status lsq_state_dequantize(const lsq_state* st, float* S, void* stream);

/* Declare that the bound scale buffer already holds frozen scales (resuming a
 * persistent-policy state from a copy of its buffers). */
lsq_status lsq_state_set_calibrated(lsq_state* st, int32_t calibrated);

/* The handle's step index t: the sequence position the next step uses for
 * dithered rounding.  It starts at 0 (lsq_state_alloc, lsq_state_zero) and
 * advances by one per step (lsq_decode_run: by H), whatever the rounding.
 * A checkpoint restores it with lsq_state_set_step_index (t >= 0, else
 * INVALID_ARG).  Host-only calls, no device work. */
lsq_status lsq_state_step_index(const lsq_state* st, int64_t* t);
lsq_status lsq_state_set_step_index(lsq_state* st, int64_t t);

/* One decode step for all heads (shapes above): Eq. (1) of "LinQuant:
 * Functional Invariances for Low-Precision Linear Recurrences" (Theoretical
 * Foundation) applied to the dequantised state, the output read from the
 * updated fp32 state, and the state requantised under the handle's scale
 * policy and rounding, as "When Dynamic Scaling Fails" (abstract) describes
 * the per-token requantisation of the decode step; the arithmetic contract at
 * the top of this file states every operation.  alpha has [heads] or
 * [heads][Dk] entries by the decay flag.  o_ref may be NULL; it is written
 * only by the yoked policy.  The state is updated in place and the handle's
 * step index advances by one.
 *
 * Ownership and errors: every pointer is a device pointer the caller owns;
 * nothing is retained after the call returns (the launch is asynchronous on
 * stream).  INVALID_ARG for a null handle or data pointer, or one that is not
 * 16-byte aligned (q, k, a diagonal alpha) or 4-byte aligned (v, a scalar
 * alpha, beta, o); NOT_CALIBRATED for a persistent-policy handle that was never
 * calibrated; HIP for a launch failure.
 *
 * HIP graphs: the launch allocates nothing and records no memset, so it can be
 * captured.  The step index, and with it the dither's sequence positions, the
 * bypass slot that is filled and which of the two b copies is read, is taken
 * from the handle on the host when the launch is issued: a captured launch
 * keeps the values of the step it was captured at.  Replaying a captured
 * sequence therefore redoes those same steps (same positions, same slots); to
 * advance a decode with a graph, capture as many steps as one replay should
 * take and, for the bypass, a whole number of merge periods starting at a
 * period boundary, and set the handle's step index (lsq_state_set_step_index)
 * to what the replays have reached before issuing further uncaptured steps. */
lsq_status lsq_decode_step(lsq_state* st, const float* q, const float* k, const float* v,
                           const float* alpha, const float* beta, float* o, float* o_ref,
                           void* stream);

/* H sequential decode steps over a decode horizon H: the state is rewritten
 * and requantised at every step of the horizon ("When Dynamic Scaling Fails",
 * abstract: the requantisation happens per token, and its effect is measured
 * against the horizon H), each step exactly lsq_decode_step.  Every input
 * carries a leading [H] axis (contiguous, step-major), o (and o_ref) receive
 * [H][heads][Dv].  The state round-trips through device memory every step; H
 * kernel launches are issued on stream; the step index advances by H.  H = 0
 * or no heads: nothing is launched.  Errors as lsq_decode_step (a negative H
 * is INVALID_ARG); a launch failure part-way returns HIP with the earlier
 * steps issued. */
lsq_status lsq_decode_run(lsq_state* st, int32_t H, const float* q, const float* k,
                          const float* v, const float* alpha, const float* beta, float* o,
                          float* o_ref, void* stream);

/* Chunkwise prefill of T tokens (linear write, no readout), after the
 * low-precision chunkwise realisation in the Methodology of "LinQuant:
 * Functional Invariances for Low-Precision Linear Recurrences".  Tokens are
 * taken in chunks of 64 (the last one may be shorter).  Per chunk and head:
 *   Gamma->_t  product of the decays of the chunk's later tokens (fp32, from
 *              the chunk's end; the diagonal decay per column),
 *   gamma^C    the product over the whole chunk,
 *   H          = Q(beta v)^T Q(Gamma-> (.) k): each operand block ([tokens x
 *              Dv] and [tokens x Dk]) is quantised to INT8 with one absmax
 *              scale s = max|x| / 127 and round-half-even codes; the integer
 *              product is exact and H = fl(h * fl(s_V * s_K)),
 *   X          = fma(gamma^C, S, H), requantised in the state's own group
 *              format and policy with round-half-even (a dynamic scale
 *              rounded to the stored scale format first, as in the decode
 *              step); the dequantised state fl(code * s) is carried to the
 *              next chunk.
 * Inputs carry a leading [T] axis (contiguous, token-major): k [T][heads][Dk],
 * v [T][heads][Dv], alpha [T][heads] (or [T][heads][Dk] for a diagonal
 * decay), beta [T][heads]; device pointers, 4-byte aligned, read-only.
 * Supported: bits 4 and 8; policy DYNAMIC or PERSISTENT (calibrated first);
 * delta 0 (the delta-rule write is sequential per token: use
 * lsq_decode_run); no bypass (lrb_rank 0); group scales along Dk (group >=
 * Dk / 8) in any stored format, or one scale per head (group 0: a dynamic
 * head scale is taken over all of the head's X at every chunk); Dk and Dv in
 * {64, 128}; otherwise UNSUPPORTED.  The state pass rounds half to even whatever the
 * handle's rounding field says.  T = 0 or no heads: nothing to do.  The step
 * index advances by T.  One workgroup per head walks the chunks in order. */
lsq_status lsq_prefill(lsq_state* st, int32_t T, const float* k, const float* v,
                       const float* alpha, const float* beta, void* stream);

/* Static description of a status code. */
const char* lsq_status_string(lsq_status s);

/* Detail of the last failing call on the calling thread ("" if none). */
const char* lsq_last_error(void);

/* Library version, major*10000 + minor*100 + patch. */
int32_t lsq_version(void);

#ifdef __cplusplus
}
#endif
#endif /* LSQ_H */
