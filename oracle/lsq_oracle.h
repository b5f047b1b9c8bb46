/*
 * CPU oracle for the low-bit recurrent-state decode step — TEST INFRASTRUCTURE.
 *
 * Only tests/, the smoke check and the benchmark's CPU-baseline leg may load
 * this library.  The product path (the HIP library) never links, includes or
 * calls anything here, and this file includes nothing from the product path.
 *
 * The oracle is plain, slow and obviously correct: scalar loops, IEEE fp32
 * arithmetic where the method computes in fp32 (so that quantisation
 * decisions are taken in the same precision as on the GPU), every row dot
 * product summed in fp32 in one stated order (blocks of 32 columns by a chain
 * of fused multiply-adds from zero, block sums added in adjacent pairs; the
 * pages leave the order open and this fixes it), correctly rounded fmaf from
 * libm, exact products in double for every rounding decision.
 *
 * Sources (page title, then the passage):
 *  - "LinQuant: Functional Invariances for Low-Precision Linear Recurrences"
 *    (picx.dev summary), Theoretical Foundation, Eq. (1): the general state
 *    update S_t = S_{t-1} Lambda_t (I - delta beta_t k_t k_t^T) + beta_t v_t k_t^T
 *    and its structural choices (scalar vs diagonal decay, write gate, delta
 *    correction).
 *  - "When Dynamic Scaling Fails: A Scale-State Feedback Governs
 *    Recurrent-State Quantization..." (abstract and project page): the state
 *    is requantised at every decode step with uniform group-wise INT4; the
 *    per-token dynamic scale is read from the state being quantised; the
 *    persistent (static) scale; the scale yoked to a full-precision reference
 *    run alongside (the same quantiser; only the source of the scale
 *    changes).
 *  - "Preserving Updates in Low-Bit Recurrent State Quantization" (abstract):
 *    Bounded Directional Rounding rounds an element whose rounded value moved
 *    opposite to its update one step toward that update.
 *  - "Low-Discrepancy Dither for Quantized Recurrent State Caches" (listing
 *    entry): a deterministic golden-ratio Weyl dither, no random numbers,
 *    replaces plain rounding of the recurrent state.  The entry fixes nothing
 *    else; the reading implemented here (LSQO_ROUND_DITHER): the code is
 *    clamp(floor(S*inv + u)), u the Weyl sequence frac(i * (sqrt(5)-1)/2)
 *    taken in 32-bit fixed point (w = i * 0x9E3779B9 mod 2^32) and truncated
 *    to 23 bits (u = (w >> 9) * 2^-23), i = step * Dv * Dk + r * Dk + c the
 *    element's position in one sequence that runs through the head's state
 *    row by row, step after step (i taken mod 2^32).
 *  - "Preserving Updates in Low-Bit Recurrent State Quantization" (abstract):
 *    Low-Rank Bypass collects small updates in a low-rank buffer and, from
 *    time to time, moves the parts of it that have grown large enough into
 *    the state.
 *    Rank, period, threshold and precision are unstated; the reading
 *    implemented here (lsqo_step_lrb): an fp32 buffer of r rank-one slots
 *    (a_j in R^Dv, b_j in R^Dk), B = sum_j a_j b_j^T, decayed with the state
 *    (scalar decay scales a_j, diagonal decay scales b_j, one fp32 product per
 *    step); each step's write w k^T goes into the next slot instead of into the
 *    quantised state, the delta projection and the readout see S' + B; every
 *    r-th step (slot r-1 written) the buffer is merged: X = S' + B built by fmas
 *    in slot order, requantised under the handle's scale policy and rounding
 *    (directional rounding takes as the update's sign the sign of the buffer
 *    value U = sum_j a_j b_j, itself built by fmas in slot order from 0), and
 *    the buffer is emptied: the elements whose code changes are the ones
 *    large enough to enter the state, the rest of the buffer is dropped.  Between
 *    merges the state is requantised from S' alone.
 *  - "LinQuant: Functional Invariances for Low-Precision Linear Recurrences"
 *    (summary page), Methodology, Low-Precision Chunkwise Realization: the
 *    state write H_[i] = Q(B_[i] V_[i])^T Q(Gamma->_[i] (.) K_[i]) and the
 *    state pass S_[i+1] = Q(gamma^C_[i] S_[i] + H_[i]) (lsqo_prefill, the
 *    linear write delta = 0).  Readings: Gamma->_t is the product of the
 *    decays of the chunk's later tokens (suffix product in fp32 from the end),
 *    gamma^C the product of all the chunk's decays; B V = fl(beta_t v_t);
 *    "Q with implicit scales" on the operands is one symmetric INT8 absmax
 *    scale per operand block (per head and chunk): s = fl(absmax/127), codes
 *    clamp(RNE(x fl(1/s))); the integer product is exact, H = fl(h fl(s_V s_K));
 *    the state pass is X = fma(gamma, S_[i], H) requantised in the state's
 *    own group format and policy with round-to-nearest-even (with one scale
 *    per head, group 0, a dynamic scale is taken over all of the head's X),
 *    and S_[i] is the dequantised state fl(C s).
 *
 * State layout used by the oracle (unpacked, host memory, heads = batch*heads):
 *   codes  int8  [heads][Dv][Dk]        signed codes in [-qmax, qmax]
 *   scales float [heads][Dv][Dk/group]  one scale per group along Dk, an fp32
 *                                       value exactly representable in the
 *                                       configured storage format
 *   ref    float [heads][Dv][Dk]        fp32 reference state (yoked policy)
 *   f32    float [heads][Dv][Dk]        fp32 state (bits == 32)
 * Inputs: q,k [heads][Dk]; v [heads][Dv]; alpha [heads] (scalar decay) or
 * [heads][Dk] (diagonal decay); beta [heads]; outputs o, o_ref [heads][Dv].
 */
#ifndef LSQ_ORACLE_H
#define LSQ_ORACLE_H
#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* enumerations (numeric values mirror the public interface by necessity) */
enum { LSQO_POLICY_NONE = 0, LSQO_POLICY_DYNAMIC = 1, LSQO_POLICY_PERSISTENT = 2, LSQO_POLICY_YOKED = 3 };
enum { LSQO_ROUND_RNE = 0, LSQO_ROUND_BDR = 1, LSQO_ROUND_DITHER = 2,
       /* rejected directional readings, for sensitivity (persistent only) */
       LSQO_ROUND_BDR_A = 3, LSQO_ROUND_BDR_B = 4 };
enum { LSQO_DECAY_SCALAR = 0, LSQO_DECAY_DIAG = 1 };
enum { LSQO_SCALE_F32 = 0, LSQO_SCALE_F16 = 1, LSQO_SCALE_BF16 = 2 };

typedef struct {
  int32_t batch, heads, dk, dv;
  int32_t bits;     /* 4, 8, or 32 (unquantised fp32 state) */
  int32_t group;    /* group size along Dk (ignored for bits == 32); 0: one scale
                       per head (dynamic or persistent, RNE or BDR, no bypass;
                       scales then hold [heads] values) */
  int32_t policy;   /* LSQO_POLICY_* */
  int32_t rounding; /* LSQO_ROUND_* */
  int32_t delta;    /* 0: linear write, 1: delta-rule correction */
  int32_t decay;    /* LSQO_DECAY_* */
  int32_t lrb_rank; /* Low-Rank Bypass slots r (0: off; lsqo_step_lrb only) */
  int32_t scale_fmt; /* LSQO_SCALE_*: stored format of the group scales (the
                        host arrays stay float, holding values of that format) */
  int64_t step;     /* sequence position of the (first) step: dithered rounding,
                       and the bypass slot (step mod r) */
} lsqo_config;

/* counters filled by a step (nullable): element-steps whose code was clamped
 * at +-qmax, and element-steps changed by directional rounding */
typedef struct {
  int64_t clamped;
  int64_t bdr_fired;
} lsqo_stats;

/* 0 on success, -1 on an invalid configuration */
int lsqo_check_config(const lsqo_config* cfg);

/* A group scale as stored in format fmt (LSQO_SCALE_*), as an fp32 value. */
float lsqo_scale_as_stored(float s, int32_t fmt);

/* One decode step for every head, in place.  o_ref (nullable) receives the
 * yoked reference readout R_t q_t. */
int lsqo_step(const lsqo_config* cfg, int8_t* codes, float* scales, float* ref, float* f32,
              const float* q, const float* k, const float* v, const float* alpha,
              const float* beta, float* o, float* o_ref, lsqo_stats* stats);

/* lsqo_step that also records, for every quantised element, the exact
 * pre-rounding values in code units: y = S_t * inv and y' = S' * inv (both
 * nullable together).  Used to decide whether a differing code lies at a
 * rounding boundary. */
int lsqo_step_trace(const lsqo_config* cfg, int8_t* codes, float* scales, float* ref,
                    float* f32, const float* q, const float* k, const float* v,
                    const float* alpha, const float* beta, float* o, float* o_ref,
                    lsqo_stats* stats, double* y_out, double* yp_out);

/* H consecutive steps; inputs carry a leading [H] dimension, o is [H][heads][Dv].
 * Heads are independent, so they are split over nthreads POSIX threads. */
int lsqo_run(const lsqo_config* cfg, int32_t H, int8_t* codes, float* scales, float* ref,
             float* f32, const float* q, const float* k, const float* v, const float* alpha,
             const float* beta, float* o, float* o_ref, int32_t nthreads);

/* One decode step with Low-Rank Bypass (cfg->lrb_rank = r >= 1; dynamic or
 * persistent policy; RNE, BDR or dithered rounding; bits 4 or 8).  Buffer
 * layout: lrb_a [heads][r][Dv], lrb_b [heads][r][Dk] fp32; slots 0 .. n-1
 * hold the buffer before the step, n = step mod r.  The step writes slot n
 * and, when n == r-1, merges (see the header note).  trace as lsqo_step_trace
 * (y_out: X*inv; yp_out: S'*inv, or the dither offset). */
int lsqo_step_lrb(const lsqo_config* cfg, int8_t* codes, float* scales, float* lrb_a,
                  float* lrb_b, const float* q, const float* k, const float* v,
                  const float* alpha, const float* beta, float* o, lsqo_stats* stats,
                  double* y_out, double* yp_out);

/* Chunkwise prefill of T tokens into the quantised state (delta = 0; dynamic
 * or persistent policy; bits 4 or 8): chunks of `chunk` tokens, the last one
 * possibly shorter.  Inputs k [T][heads][Dk], v [T][heads][Dv], alpha
 * [T][heads] or [T][heads][Dk], beta [T][heads]; codes and scales updated in
 * place (scales stay for the persistent policy); group 0: one scale per head. */
int lsqo_prefill(const lsqo_config* cfg, int32_t T, int32_t chunk, int8_t* codes, float* scales,
                 const float* k, const float* v, const float* alpha, const float* beta);

/* Quantise an fp32 state S [heads][Dv][Dk] into this configuration: one scale
 * per group from the group's absolute maximum, codes by round-to-nearest-even
 * and clamp.  The yoked policy also copies S into ref; bits == 32 copies S
 * into f32. */
int lsqo_calibrate(const lsqo_config* cfg, const float* S, int8_t* codes, float* scales,
                   float* ref, float* f32);

/* Dequantised value codes*scale, [heads][Dv][Dk] */
int lsqo_dequantize(const lsqo_config* cfg, const int8_t* codes, const float* scales, float* out);

/* Packed storage of the codes: row-major [rows][Dk*bits/8] bytes.  INT8: one
 * two's-complement byte per element.  INT4: element c of a row sits in byte
 * c/2, low nibble for even c, as a two's-complement nibble. */
int lsqo_pack(int32_t bits, int32_t dk, int64_t rows, const int8_t* codes, uint8_t* packed);
int lsqo_unpack(int32_t bits, int32_t dk, int64_t rows, const uint8_t* packed, int8_t* codes);

#ifdef __cplusplus
}
#endif
#endif
