/*
 * CPU oracle for the low-bit recurrent-state decode step — TEST INFRASTRUCTURE.
 * Plain scalar C; see lsq_oracle.h for the sources and the state layout.
 *
 * Build: gcc -std=c11 -O2 -fno-fast-math -ffp-contract=off -fPIC -shared -lm -pthread
 * (no contraction: every fused multiply-add below is an explicit fmaf, every
 * other fp32 operation rounds once, as written).
 *
 * Readings taken where the pages are silent (all stated in the design notes):
 *  - symmetric codes in [-qmax, qmax], qmax = 2^(bits-1) - 1, no zero point;
 *  - one scale per contiguous group of `group` elements along Dk, stored in
 *    fp32 or, by the configuration, rounded to nearest-even binary16 or
 *    bfloat16; every computed scale is rounded to the stored format first and
 *    the codes are formed with the stored scale;
 *  - the decay is folded into the group scale before dequantisation:
 *      S'[c] = fl(C[c] * fl(s * alpha_c));
 *  - the output is read from the fp32 state after the update and before it
 *    is requantised;
 *  - dynamic scale: fl(absmax/qmax) over the updated group; persistent: the
 *    frozen scale; yoked: fl(absmax/qmax) over the fp32 reference row after
 *    the reference's own update at the same step;
 *  - inv = fl(1/s) (0 for s == 0); codes round the exact product S*inv to
 *    nearest, ties to even, then clamp to +-qmax;
 *  - directional rounding: the update of element c is the rank-one write
 *    w*k_c, with sign sigma_c = sign(w) sign(k_c); the element "moved" from
 *    its decayed pre-write value S'[c]; both are measured in code units on
 *    the grid of this step (y = S*inv, y' = S'*inv, exact products).  A
 *    reversal is a clamped code c1 with (c1 - y') * sigma_c < 0; it is
 *    replaced by clamp(c1 + sigma_c).
 *  - dithered rounding: code = clamp(floor(S*inv + u)) with the golden-ratio
 *    Weyl offset u of the element (see lsq_oracle.h for the sequence).
 */
#include "lsq_oracle.h"

#include <math.h>
#include <pthread.h>
#include <stdlib.h>
#include <string.h>

static int qmax_of(int bits) { return (1 << (bits - 1)) - 1; }

int lsqo_check_config(const lsqo_config* cfg) {
  if (!cfg) return -1;
  if (cfg->batch < 0 || cfg->heads < 0 || cfg->dk <= 0 || cfg->dv <= 0) return -1;
  if (cfg->delta != 0 && cfg->delta != 1) return -1;
  if (cfg->decay != LSQO_DECAY_SCALAR && cfg->decay != LSQO_DECAY_DIAG) return -1;
  if (cfg->bits == 32) return (cfg->policy == LSQO_POLICY_NONE && cfg->scale_fmt == 0) ? 0 : -1;
  if (cfg->bits != 4 && cfg->bits != 8) return -1;
  if (cfg->group == 0) {
    /* one scale per head: dynamic or persistent, RNE or BDR, no bypass */
    if (cfg->policy != LSQO_POLICY_DYNAMIC && cfg->policy != LSQO_POLICY_PERSISTENT) return -1;
    if (cfg->rounding != LSQO_ROUND_RNE && cfg->rounding != LSQO_ROUND_BDR) return -1;
    if (cfg->lrb_rank != 0) return -1;
  } else if (cfg->group < 0 || cfg->dk % cfg->group != 0) {
    return -1;
  }
  if (cfg->bits == 4 && cfg->dk % 2 != 0) return -1;
  if (cfg->policy != LSQO_POLICY_DYNAMIC && cfg->policy != LSQO_POLICY_PERSISTENT &&
      cfg->policy != LSQO_POLICY_YOKED)
    return -1;
  if (cfg->rounding != LSQO_ROUND_RNE && cfg->rounding != LSQO_ROUND_BDR &&
      cfg->rounding != LSQO_ROUND_DITHER && cfg->rounding != LSQO_ROUND_BDR_A &&
      cfg->rounding != LSQO_ROUND_BDR_B)
    return -1;
  /* the rejected directional readings compare with the stored code, which lies
   * on this step's grid only under a frozen scale */
  if ((cfg->rounding == LSQO_ROUND_BDR_A || cfg->rounding == LSQO_ROUND_BDR_B) &&
      (cfg->policy != LSQO_POLICY_PERSISTENT || cfg->lrb_rank != 0))
    return -1;
  if (cfg->lrb_rank < 0) return -1;
  if (cfg->scale_fmt != LSQO_SCALE_F32 && cfg->scale_fmt != LSQO_SCALE_F16 &&
      cfg->scale_fmt != LSQO_SCALE_BF16)
    return -1;
  return 0;
}

/* round half to even of an exactly represented double */
static double round_half_even(double y) {
  double r = floor(y);
  double frac = y - r; /* exact: y has at most 48 significant bits here */
  if (frac > 0.5) return r + 1.0;
  if (frac < 0.5) return r;
  return (fmod(r, 2.0) == 0.0) ? r : r + 1.0;
}

/* 2^32 times the golden-ratio conjugate (sqrt(5)-1)/2 = 0.6180339887..., truncated */
#define LSQO_WEYL_STEP 0x9E3779B9u

/* Weyl dither of element (r, c) of a head at sequence position `step`:
 * frac(i * 0.618...) in 32-bit fixed point, truncated to 23 bits. */
/* A group scale as it is stored, returned as the fp32 value it represents:
 * fp32 unchanged; binary16 keeps 11 significant bits (quantum 2^(e-10) in the
 * binade [2^e, 2^(e+1)), e >= -14, so 2^-24 below 2^-14) rounded to nearest,
 * ties to even, and values beyond 65504 after rounding become infinity;
 * bfloat16 keeps the upper 16 bits of the fp32 pattern, rounded to nearest,
 * ties to even on the discarded 16 bits. */
static float scale_as_stored(float s, int fmt) {
  if (fmt == LSQO_SCALE_F16) {
    if (s == 0.0f || !isfinite(s)) return s;
    int e;
    frexp((double)s, &e);                       /* |s| = m 2^e, 0.5 <= m < 1 */
    const int lowest = (e - 1 < -14 ? -14 : e - 1) - 10;   /* exponent of the last kept bit */
    const double v = ldexp(round_half_even(ldexp((double)s, -lowest)), lowest);
    return fabs(v) > 65504.0 ? copysignf(INFINITY, s) : (float)v;
  }
  if (fmt == LSQO_SCALE_BF16) {
    uint32_t u;
    memcpy(&u, &s, sizeof u);
    if ((u & 0x7F800000u) == 0x7F800000u) return s;       /* infinity or NaN */
    uint32_t keep = u >> 16;
    const uint32_t rest = u & 0xFFFFu;
    if (rest > 0x8000u || (rest == 0x8000u && (keep & 1u))) keep += 1u;
    u = keep << 16;
    float r;
    memcpy(&r, &u, sizeof r);
    return r;
  }
  return s;
}

float lsqo_scale_as_stored(float s, int32_t fmt) { return scale_as_stored(s, fmt); }

static double weyl_dither(int64_t step, int dv, int dk, int r, int c) {
  const uint32_t i = (uint32_t)((uint64_t)step * (uint64_t)dv * (uint64_t)dk +
                                (uint64_t)r * (uint64_t)dk + (uint64_t)c);
  const uint32_t w = i * LSQO_WEYL_STEP; /* mod 2^32 */
  return (double)(w >> 9) * 0x1p-23;
}

static double clampd(double x, double lo, double hi) { return x < lo ? lo : (x > hi ? hi : x); }

static int sign_f(float x) { return (x > 0.0f) - (x < 0.0f); }

/* A row dot product sum_c a[c] b[c] in fp32, in the one summation order this
 * library fixes for every dot of the step (the pages leave the order open;
 * fixing it makes the codes, which depend on the delta projection, and the
 * outputs reproducible bit for bit): the columns are taken in consecutive
 * blocks of 32; inside a block the products accumulate by a chain of fused
 * multiply-adds from zero, in column order; then the block sums are added in
 * adjacent pairs, level by level ((b0 + b1) + (b2 + b3) for four blocks; an
 * unpaired last block passes to the next level as it is). */
static float dot_blocked(const float* a, const float* b, int n) {
  enum { BLOCK = 32, MAXB = 64 };
  float part[MAXB];
  int nb = 0;
  for (int c0 = 0; c0 < n; c0 += BLOCK) {
    const int c1 = (c0 + BLOCK < n) ? c0 + BLOCK : n;
    float p = 0.0f;
    for (int c = c0; c < c1; ++c) p = fmaf(a[c], b[c], p);
    part[nb++] = p;
  }
  if (nb == 0) return 0.0f;
  while (nb > 1) {
    int m = 0;
    for (int i = 0; i + 1 < nb; i += 2) part[m++] = part[i] + part[i + 1];
    if (nb % 2) part[m++] = part[nb - 1];
    nb = m;
  }
  return part[0];
}

/* Eq. (1) for one row of an fp32 state (the unquantised mode, and the yoked
 * reference).  row is updated in place; returns o_r = S_t,r . q. */
static float fp32_row_update(const lsqo_config* cfg, float* row, const float* q, const float* k,
                             float v_r, const float* alpha, float beta, float* scratch) {
  const int dk = cfg->dk;
  /* S' = S_{t-1} Lambda_t: scalar decay scales the whole row, diagonal decay
   * scales column c by alpha_c */
  for (int c = 0; c < dk; ++c) {
    float a = (cfg->decay == LSQO_DECAY_DIAG) ? alpha[c] : alpha[0];
    scratch[c] = row[c] * a;
  }
  /* delta correction: u = S' k (the part of the state aligned with k) */
  const float u = cfg->delta ? dot_blocked(scratch, k, dk) : 0.0f;
  /* S_t = S' (I - delta beta k k^T) + beta v k^T = S' + w k^T, w = beta (v - delta u) */
  float w = beta * (v_r - u);
  for (int c = 0; c < dk; ++c) row[c] = fmaf(w, k[c], scratch[c]);
  return dot_blocked(row, q, dk);
}

typedef struct {
  const lsqo_config* cfg;
  int64_t h0, h1;
  int8_t* codes;
  float* scales;
  float* ref;
  float* f32;
  const float *q, *k, *v, *alpha, *beta;
  float *o, *o_ref;
  double *y_out, *yp_out; /* nullable: exact code-unit values before rounding */
  lsqo_stats stats;
} step_job;

/* One head whose state has a single scale (group == 0, the per-head
 * granularity): every row is updated first and S_t kept whole; the scale is
 * taken over all of S_t (dynamic: fl(absmax/qmax) rounded to the stored
 * format) or kept (persistent); then every element is requantised as in the
 * group case, with directional rounding measured from S' as there. */
static void step_head_scale(step_job* J, int64_t h, const float* q, const float* k,
                            const float* v, const float* alpha, float beta) {
  const lsqo_config* cfg = J->cfg;
  const int dk = cfg->dk, dv = cfg->dv, qm = qmax_of(cfg->bits);
  const int diag = cfg->decay == LSQO_DECAY_DIAG;
  int8_t* C = J->codes + h * (int64_t)dv * dk;
  float* s = J->scales + h;
  float* SP = (float*)malloc(sizeof(float) * (size_t)dv * dk);
  float* ST = (float*)malloc(sizeof(float) * (size_t)dv * dk);
  float* W = (float*)malloc(sizeof(float) * (size_t)dv);
  float amax = 0.0f;
  for (int r = 0; r < dv; ++r) {
    float* sp = SP + (int64_t)r * dk;
    float* st = ST + (int64_t)r * dk;
    for (int c = 0; c < dk; ++c) {
      const float m = s[0] * (diag ? alpha[c] : alpha[0]);
      sp[c] = (float)C[(int64_t)r * dk + c] * m;
    }
    const float u = cfg->delta ? dot_blocked(sp, k, dk) : 0.0f;
    const float w = beta * (v[r] - u);
    W[r] = w;
    for (int c = 0; c < dk; ++c) {
      st[c] = fmaf(w, k[c], sp[c]);
      const float a = fabsf(st[c]);
      if (a > amax) amax = a;
    }
    J->o[h * dv + r] = dot_blocked(st, q, dk);
  }
  const float snew = (cfg->policy == LSQO_POLICY_PERSISTENT)
                         ? s[0] : scale_as_stored(amax / (float)qm, cfg->scale_fmt);
  const float inv = (snew == 0.0f) ? 0.0f : 1.0f / snew;
  for (int r = 0; r < dv; ++r) {
    for (int c = 0; c < dk; ++c) {
      const int64_t i = (int64_t)r * dk + c;
      const double y = (double)ST[i] * (double)inv;    /* exact */
      const double yp = (double)SP[i] * (double)inv;   /* exact */
      if (J->y_out) {
        J->y_out[h * (int64_t)dv * dk + i] = y;
        J->yp_out[h * (int64_t)dv * dk + i] = yp;
      }
      const double c0 = round_half_even(y);
      const double c1 = clampd(c0, -qm, qm);
      if (c1 != c0) J->stats.clamped++;
      double c2 = c1;
      if (cfg->rounding == LSQO_ROUND_BDR) {
        const int sigma = sign_f(W[r]) * sign_f(k[c]);
        if ((sigma > 0 && c1 < yp) || (sigma < 0 && c1 > yp)) {
          c2 = clampd(c1 + sigma, -qm, qm);
          if (c2 != c1) J->stats.bdr_fired++;
        }
      }
      C[i] = (int8_t)c2;
    }
  }
  s[0] = snew;
  free(SP);
  free(ST);
  free(W);
}

static void step_heads(step_job* J) {
  const lsqo_config* cfg = J->cfg;
  const int dk = cfg->dk, dv = cfg->dv;
  const int diag = cfg->decay == LSQO_DECAY_DIAG;
  float* sp = (float*)malloc(sizeof(float) * (size_t)dk);   /* S' */
  float* st = (float*)malloc(sizeof(float) * (size_t)dk);   /* S_t */
  float* tmp = (float*)malloc(sizeof(float) * (size_t)dk);  /* fp32 scratch */
  for (int64_t h = J->h0; h < J->h1; ++h) {
    const float* q = J->q + h * dk;
    const float* k = J->k + h * dk;
    const float* v = J->v + h * dv;
    const float* alpha = J->alpha + (diag ? h * dk : h);
    const float beta = J->beta[h];

    if (cfg->bits == 32) {
      for (int r = 0; r < dv; ++r) {
        float* row = J->f32 + (h * dv + r) * (int64_t)dk;
        J->o[h * dv + r] = fp32_row_update(cfg, row, q, k, v[r], alpha, beta, tmp);
      }
      continue;
    }

    if (cfg->group == 0) {
      step_head_scale(J, h, q, k, v, alpha, beta);
      continue;
    }
    const int g = cfg->group, ng = dk / g;
    const int qm = qmax_of(cfg->bits);
    for (int r = 0; r < dv; ++r) {
      int8_t* C = J->codes + (h * dv + r) * (int64_t)dk;
      float* s = J->scales + (h * dv + r) * (int64_t)ng;

      /* yoked arm: advance the fp32 reference row first (same inputs) */
      float* R = NULL;
      if (cfg->policy == LSQO_POLICY_YOKED) {
        R = J->ref + (h * dv + r) * (int64_t)dk;
        float oref = fp32_row_update(cfg, R, q, k, v[r], alpha, beta, tmp);
        if (J->o_ref) J->o_ref[h * dv + r] = oref;
      }

      /* dequantise with the decay folded into the group scale */
      for (int c = 0; c < dk; ++c) {
        float a = diag ? alpha[c] : alpha[0];
        float m = s[c / g] * a;
        sp[c] = (float)C[c] * m;
      }
      const float u = cfg->delta ? dot_blocked(sp, k, dk) : 0.0f;
      float w = beta * (v[r] - u);
      for (int c = 0; c < dk; ++c) st[c] = fmaf(w, k[c], sp[c]);
      J->o[h * dv + r] = dot_blocked(st, q, dk);

      /* scale policy, then requantise group by group */
      for (int gi = 0; gi < ng; ++gi) {
        float snew;
        if (cfg->policy == LSQO_POLICY_PERSISTENT) {
          snew = s[gi];
        } else {
          const float* src = (cfg->policy == LSQO_POLICY_YOKED) ? R : st;
          float amax = 0.0f;
          for (int c = gi * g; c < (gi + 1) * g; ++c) {
            float a = fabsf(src[c]);
            if (a > amax) amax = a;
          }
          snew = scale_as_stored(amax / (float)qm, cfg->scale_fmt);
        }
        float inv = (snew == 0.0f) ? 0.0f : 1.0f / snew;
        for (int c = gi * g; c < (gi + 1) * g; ++c) {
          double y = (double)st[c] * (double)inv; /* exact */
          if (J->y_out) {
            J->y_out[(h * dv + r) * (int64_t)dk + c] = y;
            J->yp_out[(h * dv + r) * (int64_t)dk + c] = (double)sp[c] * (double)inv;
          }
          double c0;
          if (cfg->rounding == LSQO_ROUND_DITHER) {
            /* floor(y + u), decided exactly: y - floor(y) and 1 - u are exact
             * (y has at most 48 significant bits, u 23 bits below the point) */
            const double u = weyl_dither(cfg->step, dv, dk, r, c);
            const double fy = floor(y);
            c0 = fy + ((y - fy >= 1.0 - u) ? 1.0 : 0.0);
            if (J->yp_out) J->yp_out[(h * dv + r) * (int64_t)dk + c] = u;
          } else {
            c0 = round_half_even(y);
          }
          double c1 = clampd(c0, -qm, qm);
          if (c1 != c0) J->stats.clamped++;
          double c2 = c1;
          if (cfg->rounding == LSQO_ROUND_BDR) {
            int sigma = sign_f(w) * sign_f(k[c]);
            double yp = (double)sp[c] * (double)inv; /* exact */
            int reversed = (sigma > 0 && c1 < yp) || (sigma < 0 && c1 > yp);
            if (reversed) {
              c2 = clampd(c1 + sigma, -qm, qm);
              if (c2 != c1) J->stats.bdr_fired++;
            }
          } else if (cfg->rounding == LSQO_ROUND_BDR_A || cfg->rounding == LSQO_ROUND_BDR_B) {
            /* The two readings of directional rounding that were not taken,
             * kept for sensitivity (frozen scale: the stored value C_old s is
             * code C_old on this step's grid).  A: the update is the total
             * change from the stored value, sigma = sign(S - C_old s) (the
             * sign of a rounded double difference is exact).  B': the update
             * is the rank-one write (sigma as above), the move is measured
             * from the stored value.  Reversal: c1 on the far side of C_old. */
            const double cold = (double)C[c];
            int sigma;
            if (cfg->rounding == LSQO_ROUND_BDR_A) {
              const double d = (double)st[c] - cold * (double)snew;
              sigma = (d > 0.0) - (d < 0.0);
            } else {
              sigma = sign_f(w) * sign_f(k[c]);
            }
            const int reversed = snew > 0.0f && ((sigma > 0 && c1 < cold) || (sigma < 0 && c1 > cold));
            if (reversed) {
              c2 = clampd(c1 + sigma, -qm, qm);
              if (c2 != c1) J->stats.bdr_fired++;
            }
          }
          C[c] = (int8_t)c2;
        }
        s[gi] = snew;
      }
    }
  }
  free(sp);
  free(st);
  free(tmp);
}

int lsqo_step(const lsqo_config* cfg, int8_t* codes, float* scales, float* ref, float* f32,
              const float* q, const float* k, const float* v, const float* alpha,
              const float* beta, float* o, float* o_ref, lsqo_stats* stats) {
  return lsqo_step_trace(cfg, codes, scales, ref, f32, q, k, v, alpha, beta, o, o_ref, stats,
                         NULL, NULL);
}

int lsqo_step_trace(const lsqo_config* cfg, int8_t* codes, float* scales, float* ref,
                    float* f32, const float* q, const float* k, const float* v,
                    const float* alpha, const float* beta, float* o, float* o_ref,
                    lsqo_stats* stats, double* y_out, double* yp_out) {
  if (lsqo_check_config(cfg)) return -1;
  if ((y_out == NULL) != (yp_out == NULL)) return -1;
  step_job J;
  memset(&J, 0, sizeof J);
  J.cfg = cfg;
  J.h0 = 0;
  J.h1 = (int64_t)cfg->batch * cfg->heads;
  J.codes = codes; J.scales = scales; J.ref = ref; J.f32 = f32;
  J.q = q; J.k = k; J.v = v; J.alpha = alpha; J.beta = beta; J.o = o; J.o_ref = o_ref;
  J.y_out = y_out; J.yp_out = yp_out;
  step_heads(&J);
  if (stats) {
    stats->clamped += J.stats.clamped;
    stats->bdr_fired += J.stats.bdr_fired;
  }
  return 0;
}

typedef struct {
  step_job job;
  int32_t H;
  int64_t n;
} run_job;

static void* run_worker(void* arg) {
  run_job* R = (run_job*)arg;
  step_job J = R->job;
  const lsqo_config* cfg = J.cfg;
  const int64_t n = R->n;
  const int64_t dk = cfg->dk, dv = cfg->dv;
  const int64_t astride = (cfg->decay == LSQO_DECAY_DIAG) ? n * dk : n;
  lsqo_config ct = *cfg;
  J.cfg = &ct;
  for (int32_t t = 0; t < R->H; ++t) {
    ct.step = cfg->step + t;
    J.q = R->job.q + t * n * dk;
    J.k = R->job.k + t * n * dk;
    J.v = R->job.v + t * n * dv;
    J.alpha = R->job.alpha + t * astride;
    J.beta = R->job.beta + t * n;
    J.o = R->job.o + t * n * dv;
    J.o_ref = R->job.o_ref ? R->job.o_ref + t * n * dv : NULL;
    step_heads(&J);
  }
  R->job.stats = J.stats;
  return NULL;
}

int lsqo_run(const lsqo_config* cfg, int32_t H, int8_t* codes, float* scales, float* ref,
             float* f32, const float* q, const float* k, const float* v, const float* alpha,
             const float* beta, float* o, float* o_ref, int32_t nthreads) {
  if (lsqo_check_config(cfg) || H < 0) return -1;
  const int64_t n = (int64_t)cfg->batch * cfg->heads;
  if (nthreads < 1) nthreads = 1;
  if (nthreads > n && n > 0) nthreads = (int32_t)n;
  run_job* jobs = (run_job*)calloc((size_t)nthreads, sizeof(run_job));
  pthread_t* th = (pthread_t*)calloc((size_t)nthreads, sizeof(pthread_t));
  for (int32_t i = 0; i < nthreads; ++i) {
    step_job* J = &jobs[i].job;
    J->cfg = cfg;
    J->h0 = n * i / nthreads;
    J->h1 = n * (i + 1) / nthreads;
    J->codes = codes; J->scales = scales; J->ref = ref; J->f32 = f32;
    J->q = q; J->k = k; J->v = v; J->alpha = alpha; J->beta = beta; J->o = o; J->o_ref = o_ref;
    jobs[i].H = H;
    jobs[i].n = n;
  }
  if (nthreads == 1) {
    run_worker(&jobs[0]);
  } else {
    for (int32_t i = 0; i < nthreads; ++i) pthread_create(&th[i], NULL, run_worker, &jobs[i]);
    for (int32_t i = 0; i < nthreads; ++i) pthread_join(th[i], NULL);
  }
  free(jobs);
  free(th);
  return 0;
}

/* Requantise one group of a row from the fp32 values x (S_t, or the merged
 * X), the decayed pre-write values sp and the update signs sig (+-1, 0 for
 * none), under the configuration's rounding; returns the number of codes
 * changed by directional rounding.  Shared by the bypass step. */
static int64_t requantise_group(const lsqo_config* cfg, int r, int c0, int c1, const float* x,
                                const float* sp, const int* sig, float inv, int8_t* C,
                                lsqo_stats* stats, double* y_row, double* yp_row) {
  const int qm = qmax_of(cfg->bits);
  int64_t fired = 0;
  for (int c = c0; c < c1; ++c) {
    const double y = (double)x[c] * (double)inv;   /* exact */
    const double yp = (double)sp[c] * (double)inv; /* exact */
    if (y_row) { y_row[c] = y; yp_row[c] = yp; }
    double q0;
    if (cfg->rounding == LSQO_ROUND_DITHER) {
      const double u = weyl_dither(cfg->step, cfg->dv, cfg->dk, r, c);
      const double fy = floor(y);
      q0 = fy + ((y - fy >= 1.0 - u) ? 1.0 : 0.0);
      if (yp_row) yp_row[c] = u;
    } else {
      q0 = round_half_even(y);
    }
    double q1 = clampd(q0, -qm, qm);
    if (q1 != q0) stats->clamped++;
    double q2 = q1;
    if (cfg->rounding == LSQO_ROUND_BDR && sig[c] != 0) {
      const int sigma = sig[c];
      if ((sigma > 0 && q1 < yp) || (sigma < 0 && q1 > yp)) {
        q2 = clampd(q1 + sigma, -qm, qm);
        if (q2 != q1) fired++;
      }
    }
    C[c] = (int8_t)q2;
  }
  stats->bdr_fired += fired;
  return fired;
}

int lsqo_step_lrb(const lsqo_config* cfg, int8_t* codes, float* scales, float* lrb_a,
                  float* lrb_b, const float* q, const float* k, const float* v,
                  const float* alpha, const float* beta, float* o, lsqo_stats* stats,
                  double* y_out, double* yp_out) {
  if (lsqo_check_config(cfg) || cfg->bits == 32 || cfg->lrb_rank < 1) return -1;
  if (cfg->policy != LSQO_POLICY_DYNAMIC && cfg->policy != LSQO_POLICY_PERSISTENT) return -1;
  if ((y_out == NULL) != (yp_out == NULL)) return -1;
  const int dk = cfg->dk, dv = cfg->dv, R = cfg->lrb_rank;
  const int diag = cfg->decay == LSQO_DECAY_DIAG;
  const int g = cfg->group, ng = dk / g, qm = qmax_of(cfg->bits);
  const int n_used = (int)(cfg->step % R);   /* filled slots before this step */
  const int merge = n_used == R - 1;
  const int64_t nh = (int64_t)cfg->batch * cfg->heads;
  lsqo_stats st = {0, 0};
  float* sp = (float*)malloc(sizeof(float) * (size_t)dk);
  float* x = (float*)malloc(sizeof(float) * (size_t)dk);
  int* sig = (int*)malloc(sizeof(int) * (size_t)dk);
  float* bk = (float*)malloc(sizeof(float) * (size_t)R);
  float* bq = (float*)malloc(sizeof(float) * (size_t)R);
  for (int64_t h = 0; h < nh; ++h) {
    const float* qh = q + h * dk;
    const float* kh = k + h * dk;
    const float* ah = alpha + (diag ? h * dk : h);
    float* A = lrb_a + h * (int64_t)R * dv;   /* A[j*dv + i] = a_j[i] */
    float* Bv = lrb_b + h * (int64_t)R * dk;  /* Bv[j*dk + c] = b_j[c] */
    /* decay the buffer with the state: B' = B Lambda_t */
    for (int j = 0; j < n_used; ++j) {
      if (diag) {
        for (int c = 0; c < dk; ++c) Bv[j * dk + c] = Bv[j * dk + c] * ah[c];
      } else {
        for (int i = 0; i < dv; ++i) A[j * dv + i] = A[j * dv + i] * ah[0];
      }
    }
    /* per-slot projections b_j . k and b_j . q */
    for (int j = 0; j < n_used; ++j) {
      bk[j] = dot_blocked(Bv + j * dk, kh, dk);
      bq[j] = dot_blocked(Bv + j * dk, qh, dk);
    }
    const float kq = dot_blocked(kh, qh, dk);
    /* the new slot holds k */
    for (int c = 0; c < dk; ++c) Bv[n_used * dk + c] = kh[c];

    for (int i = 0; i < dv; ++i) {
      int8_t* C = codes + (h * dv + i) * (int64_t)dk;
      float* s = scales + (h * dv + i) * (int64_t)ng;
      for (int c = 0; c < dk; ++c) {
        float a = diag ? ah[c] : ah[0];
        float m = s[c / g] * a;
        sp[c] = (float)C[c] * m;
      }
      /* delta projection on the effective state S' + B' */
      float u = 0.0f;
      if (cfg->delta) {
        /* S'.k, then the slots' a_j (b_j.k) in slot order */
        u = dot_blocked(sp, kh, dk);
        for (int j = 0; j < n_used; ++j) u = fmaf(A[j * dv + i], bk[j], u);
      }
      const float w = beta[h] * (v[h * dv + i] - u);
      A[n_used * dv + i] = w;   /* slot n: the write w k^T */
      /* readout from S' + B' + w k^T: S'.q, the slots' a_j (b_j.q), then w (k.q) */
      float oo = dot_blocked(sp, qh, dk);
      for (int j = 0; j < n_used; ++j) oo = fmaf(A[j * dv + i], bq[j], oo);
      oo = fmaf(w, kq, oo);
      o[h * dv + i] = oo;
      /* the value to requantise: the merged X on a merge step, else S' */
      for (int c = 0; c < dk; ++c) {
        float xv = sp[c], uv = 0.0f;   /* merged value, and the buffer's own value */
        if (merge) {
          for (int j = 0; j <= n_used; ++j) {
            xv = fmaf(A[j * dv + i], Bv[j * dk + c], xv);
            uv = fmaf(A[j * dv + i], Bv[j * dk + c], uv);
          }
        }
        x[c] = xv;
        sig[c] = (uv > 0.0f) - (uv < 0.0f);   /* direction of the accumulated update */
      }
      for (int gi = 0; gi < ng; ++gi) {
        float snew;
        if (cfg->policy == LSQO_POLICY_PERSISTENT) {
          snew = s[gi];
        } else {
          float amax = 0.0f;
          for (int c = gi * g; c < (gi + 1) * g; ++c) {
            float av = fabsf(x[c]);
            if (av > amax) amax = av;
          }
          snew = scale_as_stored(amax / (float)qm, cfg->scale_fmt);
        }
        const float inv = (snew == 0.0f) ? 0.0f : 1.0f / snew;
        requantise_group(cfg, i, gi * g, (gi + 1) * g, x, sp, sig, inv, C, &st,
                         y_out ? y_out + (h * dv + i) * (int64_t)dk : NULL,
                         yp_out ? yp_out + (h * dv + i) * (int64_t)dk : NULL);
        s[gi] = snew;
      }
    }
  }
  free(sp);
  free(x);
  free(sig);
  free(bk);
  free(bq);
  if (stats) {
    stats->clamped += st.clamped;
    stats->bdr_fired += st.bdr_fired;
  }
  return 0;
}

/* symmetric INT8 absmax quantisation of a block (the chunk operands) */
static float quantise_block_i8(const float* x, int64_t n, int8_t* q) {
  float amax = 0.0f;
  for (int64_t i = 0; i < n; ++i) {
    float a = fabsf(x[i]);
    if (a > amax) amax = a;
  }
  const float s = amax / 127.0f;
  const float inv = (s == 0.0f) ? 0.0f : 1.0f / s;
  for (int64_t i = 0; i < n; ++i)
    q[i] = (int8_t)clampd(round_half_even((double)x[i] * (double)inv), -127, 127);
  return s;
}

int lsqo_prefill(const lsqo_config* cfg, int32_t T, int32_t chunk, int8_t* codes, float* scales,
                 const float* k, const float* v, const float* alpha, const float* beta) {
  if (lsqo_check_config(cfg) || cfg->bits == 32 || cfg->delta != 0 || T < 0 || chunk < 1)
    return -1;
  if (cfg->policy != LSQO_POLICY_DYNAMIC && cfg->policy != LSQO_POLICY_PERSISTENT) return -1;
  /* group 0: one scale per head, over the whole Dv x Dk state */
  const int head = cfg->group == 0;
  const int dk = cfg->dk, dv = cfg->dv, g = head ? cfg->dk : cfg->group, ng = dk / g;
  const int qm = qmax_of(cfg->bits);
  const int diag = cfg->decay == LSQO_DECAY_DIAG;
  const int64_t nh = (int64_t)cfg->batch * cfg->heads;
  const int da = diag ? dk : 1;                 /* decay values per token */
  float* S = (float*)malloc(sizeof(float) * (size_t)dv * dk);     /* dequantised state */
  float* G = (float*)malloc(sizeof(float) * (size_t)chunk * da);  /* Gamma-> per token */
  float* gam = (float*)malloc(sizeof(float) * (size_t)da);        /* gamma^C */
  float* BV = (float*)malloc(sizeof(float) * (size_t)chunk * dv);
  float* GK = (float*)malloc(sizeof(float) * (size_t)chunk * dk);
  int8_t* Vq = (int8_t*)malloc((size_t)chunk * dv);
  int8_t* Kq = (int8_t*)malloc((size_t)chunk * dk);
  for (int64_t h = 0; h < nh; ++h) {
    int8_t* Ch = codes + h * (int64_t)dv * dk;
    float* sh = head ? scales + h : scales + h * (int64_t)dv * ng;
    for (int r = 0; r < dv; ++r)
      for (int c = 0; c < dk; ++c)
        S[r * dk + c] = (float)Ch[r * dk + c] * sh[head ? 0 : r * ng + c / g];
    for (int32_t t0 = 0; t0 < T; t0 += chunk) {
      const int tc = (T - t0 < chunk) ? (int)(T - t0) : chunk;
      /* decay products: Gamma->_t = prod_{s>t} alpha_s within the chunk */
      for (int a = 0; a < da; ++a) {
        float acc = 1.0f;
        for (int t = tc - 1; t >= 0; --t) {
          G[t * da + a] = acc;
          const float* at = alpha + ((int64_t)(t0 + t) * nh + h) * da;
          acc = acc * at[a];
        }
        gam[a] = acc;
      }
      /* chunk operands */
      for (int t = 0; t < tc; ++t) {
        const int64_t row = (int64_t)(t0 + t) * nh + h;
        const float b = beta[row];
        for (int i = 0; i < dv; ++i) BV[t * dv + i] = b * v[row * dv + i];
        for (int c = 0; c < dk; ++c) GK[t * dk + c] = G[t * da + (diag ? c : 0)] * k[row * dk + c];
      }
      const float s_v = quantise_block_i8(BV, (int64_t)tc * dv, Vq);
      const float s_k = quantise_block_i8(GK, (int64_t)tc * dk, Kq);
      const float sc = s_v * s_k;
      if (head) {
        /* one scale per head: every element of X first, then the head's
         * absmax (dynamic), then the codes */
        float amax = 0.0f;
        for (int r = 0; r < dv; ++r) {
          float* x = S + r * dk;
          for (int c = 0; c < dk; ++c) {
            int64_t hacc = 0;
            for (int t = 0; t < tc; ++t) hacc += (int64_t)Vq[t * dv + r] * (int64_t)Kq[t * dk + c];
            const float H = (float)hacc * sc;
            x[c] = fmaf(gam[diag ? c : 0], x[c], H);
            const float a = fabsf(x[c]);
            if (a > amax) amax = a;
          }
        }
        float snew = sh[0];
        if (cfg->policy == LSQO_POLICY_DYNAMIC) snew = scale_as_stored(amax / (float)qm, cfg->scale_fmt);
        const float inv = (snew == 0.0f) ? 0.0f : 1.0f / snew;
        for (int64_t i = 0; i < (int64_t)dv * dk; ++i) {
          const double q = clampd(round_half_even((double)S[i] * (double)inv), -qm, qm);
          Ch[i] = (int8_t)q;
          S[i] = (float)q * snew;
        }
        sh[0] = snew;
        continue;
      }
      /* state pass, row by row */
      for (int r = 0; r < dv; ++r) {
        float* x = S + r * dk;
        for (int c = 0; c < dk; ++c) {
          int64_t hacc = 0;
          for (int t = 0; t < tc; ++t) hacc += (int64_t)Vq[t * dv + r] * (int64_t)Kq[t * dk + c];
          const float H = (float)hacc * sc;
          x[c] = fmaf(gam[diag ? c : 0], x[c], H);
        }
        for (int gi = 0; gi < ng; ++gi) {
          float snew = sh[r * ng + gi];
          if (cfg->policy == LSQO_POLICY_DYNAMIC) {
            float amax = 0.0f;
            for (int c = gi * g; c < (gi + 1) * g; ++c) {
              float a = fabsf(x[c]);
              if (a > amax) amax = a;
            }
            snew = scale_as_stored(amax / (float)qm, cfg->scale_fmt);
          }
          const float inv = (snew == 0.0f) ? 0.0f : 1.0f / snew;
          for (int c = gi * g; c < (gi + 1) * g; ++c) {
            const double q = clampd(round_half_even((double)x[c] * (double)inv), -qm, qm);
            Ch[r * dk + c] = (int8_t)q;
            x[c] = (float)q * snew;   /* the dequantised state carried to the next chunk */
          }
          sh[r * ng + gi] = snew;
        }
      }
    }
  }
  free(S); free(G); free(gam); free(BV); free(GK); free(Vq); free(Kq);
  return 0;
}

int lsqo_calibrate(const lsqo_config* cfg, const float* S, int8_t* codes, float* scales,
                   float* ref, float* f32) {
  if (lsqo_check_config(cfg)) return -1;
  const int64_t n = (int64_t)cfg->batch * cfg->heads;
  const int64_t rows = n * cfg->dv;
  const int dk = cfg->dk;
  if (cfg->bits == 32) {
    memcpy(f32, S, sizeof(float) * (size_t)(rows * dk));
    return 0;
  }
  if (cfg->group == 0) {                      /* one scale per head */
    const int64_t per = (int64_t)cfg->dv * dk;
    const int qmh = qmax_of(cfg->bits);
    for (int64_t h = 0; h < n; ++h) {
      const float* x = S + h * per;
      float amax = 0.0f;
      for (int64_t i = 0; i < per; ++i) {
        const float a = fabsf(x[i]);
        if (a > amax) amax = a;
      }
      const float s = scale_as_stored(amax / (float)qmh, cfg->scale_fmt);
      const float inv = (s == 0.0f) ? 0.0f : 1.0f / s;
      for (int64_t i = 0; i < per; ++i)
        codes[h * per + i] = (int8_t)clampd(round_half_even((double)x[i] * (double)inv), -qmh, qmh);
      scales[h] = s;
    }
    return 0;
  }
  const int g = cfg->group, ng = dk / g, qm = qmax_of(cfg->bits);
  for (int64_t r = 0; r < rows; ++r) {
    const float* x = S + r * dk;
    for (int gi = 0; gi < ng; ++gi) {
      float amax = 0.0f;
      for (int c = gi * g; c < (gi + 1) * g; ++c) {
        float a = fabsf(x[c]);
        if (a > amax) amax = a;
      }
      float s = scale_as_stored(amax / (float)qm, cfg->scale_fmt);
      float inv = (s == 0.0f) ? 0.0f : 1.0f / s;
      for (int c = gi * g; c < (gi + 1) * g; ++c) {
        double y = (double)x[c] * (double)inv;
        codes[r * dk + c] = (int8_t)clampd(round_half_even(y), -qm, qm);
      }
      scales[r * ng + gi] = s;
    }
  }
  if (cfg->policy == LSQO_POLICY_YOKED) memcpy(ref, S, sizeof(float) * (size_t)(rows * dk));
  return 0;
}

int lsqo_dequantize(const lsqo_config* cfg, const int8_t* codes, const float* scales, float* out) {
  if (lsqo_check_config(cfg) || cfg->bits == 32) return -1;
  const int64_t rows = (int64_t)cfg->batch * cfg->heads * cfg->dv;
  const int dk = cfg->dk;
  if (cfg->group == 0) {                      /* one scale per head */
    for (int64_t r = 0; r < rows; ++r)
      for (int c = 0; c < dk; ++c) out[r * dk + c] = (float)codes[r * dk + c] * scales[r / cfg->dv];
    return 0;
  }
  const int g = cfg->group, ng = dk / g;
  for (int64_t r = 0; r < rows; ++r)
    for (int c = 0; c < dk; ++c) out[r * dk + c] = (float)codes[r * dk + c] * scales[r * ng + c / g];
  return 0;
}

int lsqo_pack(int32_t bits, int32_t dk, int64_t rows, const int8_t* codes, uint8_t* packed) {
  if (bits == 8) {
    for (int64_t i = 0; i < rows * dk; ++i) packed[i] = (uint8_t)codes[i];
    return 0;
  }
  if (bits != 4 || dk % 2) return -1;
  for (int64_t r = 0; r < rows; ++r)
    for (int c = 0; c < dk; c += 2) {
      uint8_t lo = (uint8_t)codes[r * dk + c] & 0x0F;
      uint8_t hi = (uint8_t)codes[r * dk + c + 1] & 0x0F;
      packed[r * (dk / 2) + c / 2] = (uint8_t)(lo | (hi << 4));
    }
  return 0;
}

static int8_t sext4(unsigned nib) { return (int8_t)((nib & 0x8) ? (int)nib - 16 : (int)nib); }

int lsqo_unpack(int32_t bits, int32_t dk, int64_t rows, const uint8_t* packed, int8_t* codes) {
  if (bits == 8) {
    for (int64_t i = 0; i < rows * dk; ++i) codes[i] = (int8_t)packed[i];
    return 0;
  }
  if (bits != 4 || dk % 2) return -1;
  for (int64_t r = 0; r < rows; ++r)
    for (int c = 0; c < dk; c += 2) {
      uint8_t b = packed[r * (dk / 2) + c / 2];
      codes[r * dk + c] = sext4(b & 0x0F);
      codes[r * dk + c + 1] = sext4(b >> 4);
    }
  return 0;
}
