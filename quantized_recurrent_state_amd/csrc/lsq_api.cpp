// Host side of the C ABI in include/lsq.h: validation, handles, launch
// geometry and dispatch.  All device work is in the .hip translation units.
#include <hip/hip_runtime.h>

#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <new>
#include <string>

#include "lsq.h"
#include "lsq_internal.h"
#include "lsq_probe.h"

struct lsq_state {
  lsq_config cfg;
  void* codes;
  float* scales;
  float* ref;
  float* f32;
  float* lrb;
  int32_t calibrated;
  int64_t step;          // sequence position of the next step (dithered rounding)
};

namespace {

thread_local std::string g_last_error;

lsq_status fail(lsq_status s, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
lsq_status fail(lsq_status s, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return s;
}

lsq_status ok() {
  g_last_error.clear();
  return LSQ_OK;
}

int64_t n_heads(const lsq_config& c) { return (int64_t)c.batch * c.heads; }

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool aligned4(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 3u) == 0; }

// Checks that make a configuration meaningless (INVALID_ARG) and the ones this
// build has no kernel for (UNSUPPORTED).
lsq_status check_config(const lsq_config* c) {
  if (!c) return fail(LSQ_ERR_INVALID_ARG, "config is null");
  if (c->batch < 0 || c->heads < 0) return fail(LSQ_ERR_INVALID_ARG, "negative batch or heads");
  if (c->dk <= 0 || c->dv <= 0) return fail(LSQ_ERR_INVALID_ARG, "dk and dv must be positive");
  if (c->delta != 0 && c->delta != 1) return fail(LSQ_ERR_INVALID_ARG, "delta must be 0 or 1");
  if (c->decay != LSQ_DECAY_SCALAR && c->decay != LSQ_DECAY_DIAG)
    return fail(LSQ_ERR_INVALID_ARG, "decay must be SCALAR or DIAG");
  if (c->rounding != LSQ_ROUND_RNE && c->rounding != LSQ_ROUND_BDR &&
      c->rounding != LSQ_ROUND_DITHER && c->rounding != LSQ_ROUND_BDR_A &&
      c->rounding != LSQ_ROUND_BDR_B)
    return fail(LSQ_ERR_INVALID_ARG, "rounding must be RNE, BDR, DITHER, BDR_A or BDR_B");
  if ((c->rounding == LSQ_ROUND_BDR_A || c->rounding == LSQ_ROUND_BDR_B) &&
      (c->bits == 32 || c->policy != LSQ_POLICY_PERSISTENT))
    return fail(LSQ_ERR_INVALID_ARG, "BDR_A and BDR_B compare with the stored code: persistent scale only");
  if (c->bits == 32) {
    if (c->policy != LSQ_POLICY_NONE)
      return fail(LSQ_ERR_INVALID_ARG, "an fp32 state (bits 32) takes policy NONE");
  } else if (c->bits == 4 || c->bits == 8) {
    if (c->policy != LSQ_POLICY_DYNAMIC && c->policy != LSQ_POLICY_PERSISTENT &&
        c->policy != LSQ_POLICY_YOKED)
      return fail(LSQ_ERR_INVALID_ARG, "a quantised state takes policy DYNAMIC, PERSISTENT or YOKED");
    if (c->group < 0 || (c->group > 0 && c->dk % c->group != 0))
      return fail(LSQ_ERR_INVALID_ARG, "group must be 0 (one scale per head) or divide dk");
    if (c->group == 0 && (c->policy == LSQ_POLICY_YOKED || c->rounding == LSQ_ROUND_DITHER ||
                          c->rounding == LSQ_ROUND_BDR_A || c->rounding == LSQ_ROUND_BDR_B))
      return fail(LSQ_ERR_INVALID_ARG,
                  "one scale per head takes the DYNAMIC or PERSISTENT policy, RNE or BDR");
  } else {
    return fail(LSQ_ERR_INVALID_ARG, "bits must be 4, 8 or 32");
  }
  if (c->dk != 64 && c->dk != 128) return fail(LSQ_ERR_UNSUPPORTED, "dk %d: this library has dk 64 and 128", c->dk);
  if (c->bits != 32 && c->group == 0) {
    if (c->scale_fmt != LSQ_SCALE_F32 || c->lrb_rank != 0)
      return fail(LSQ_ERR_UNSUPPORTED, "one scale per head runs with an fp32 scale and no bypass");
    if (c->dv > 1024) return fail(LSQ_ERR_UNSUPPORTED, "one scale per head needs dv <= 1024");
  } else if (c->bits != 32) {
    constexpr int min_group = 16;   // a lane owns 32 elements: one group, or two of 16
    if (c->group < min_group || (c->group & (c->group - 1)) != 0)
      return fail(LSQ_ERR_UNSUPPORTED,
                  "group %d: this library needs a power-of-two group of at least %d elements",
                  c->group, min_group);
  }
  if (c->scale_fmt != LSQ_SCALE_F32 && c->scale_fmt != LSQ_SCALE_F16 &&
      c->scale_fmt != LSQ_SCALE_BF16)
    return fail(LSQ_ERR_INVALID_ARG, "scale_fmt must be F32, F16 or BF16");
  if (c->bits == 32 && c->scale_fmt != LSQ_SCALE_F32)
    return fail(LSQ_ERR_INVALID_ARG, "an fp32 state has no scales (scale_fmt F32)");
  if (c->lrb_rank < 0 || c->lrb_rank > 8)
    return fail(LSQ_ERR_INVALID_ARG, "lrb_rank must be 0 to 8");
  if (c->rounding == LSQ_ROUND_BDR_A || c->rounding == LSQ_ROUND_BDR_B) {
    if (c->group < 32 || c->scale_fmt != LSQ_SCALE_F32 || c->lrb_rank != 0)
      return fail(LSQ_ERR_UNSUPPORTED,
                  "BDR_A and BDR_B run with groups of 32 or more, fp32 scales and no bypass");
  }
  if (c->lrb_rank > 0) {
    if (c->bits == 32) return fail(LSQ_ERR_INVALID_ARG, "the bypass applies to a quantised state");
    if (c->policy != LSQ_POLICY_DYNAMIC && c->policy != LSQ_POLICY_PERSISTENT)
      return fail(LSQ_ERR_UNSUPPORTED, "the bypass supports the DYNAMIC and PERSISTENT policies");
    if (c->group < 32)
      return fail(LSQ_ERR_UNSUPPORTED, "the bypass needs groups of 32 or more elements");
    if (c->scale_fmt != LSQ_SCALE_F32)
      return fail(LSQ_ERR_UNSUPPORTED, "the bypass keeps fp32 scales");
  }
  const lsq::Geometry g = lsq::geometry(c->bits, c->dk);
  const int64_t iters = (c->dv + g.rows_per_iter - 1) / g.rows_per_iter;
  if (n_heads(*c) * iters > INT32_MAX / 2)
    return fail(LSQ_ERR_UNSUPPORTED, "batch*heads*dv too large for one launch");
  return ok();
}

constexpr int kBuffers = 5;   // codes, scales, ref, f32, lrb

void sizes_of(const lsq_config& c, size_t (&sz)[kBuffers]) {
  const size_t elems = (size_t)n_heads(c) * c.dv * c.dk;
  for (size_t& x : sz) x = 0;
  if (c.bits == 32) {
    sz[3] = elems * 4;
    return;
  }
  sz[0] = elems * c.bits / 8;
  sz[1] = (c.group == 0) ? (size_t)n_heads(c) * 4     // one fp32 scale per head
                         : (size_t)n_heads(c) * c.dv * (c.dk / c.group) *
                               (c.scale_fmt == LSQ_SCALE_F32 ? 4 : 2);
  if (c.policy == LSQ_POLICY_YOKED) sz[2] = elems * 4;
  if (c.lrb_rank > 0) sz[4] = (size_t)n_heads(c) * c.lrb_rank * (c.dv + 2 * (size_t)c.dk) * 4;
}

// Wave target of the plain quantised step (see launch_one_step).
#ifndef LSQ_LEAN_WAVES
#define LSQ_LEAN_WAVES 4096
#endif

// Launch geometry: one wave per (head, slice of nit row-iterations); slices
// shrink until there are at least `target` waves.  The default, 8192 (256 CUs
// x 32 waves), keeps every SIMD busy when a wave's rows are memory-heavy.
void choose_slices(const lsq_config& c, int32_t* nit, int32_t* wph, int32_t* total,
                   int64_t target = 8192) {
  const lsq::Geometry g = lsq::geometry(c.bits, c.dk);
  const int32_t iters = (c.dv + g.rows_per_iter - 1) / g.rows_per_iter;
  const int64_t heads = n_heads(c);
  int32_t it = iters;
  while (it > 1 && heads * ((iters + it - 1) / it) < target) it = (it + 1) / 2;
  *nit = it;
  *wph = (iters + it - 1) / it;
  *total = (int32_t)(heads * *wph);
}

lsq_status hip_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return ok();
  return fail(LSQ_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

lsq_status check_step_ptrs(const lsq_state* st, const float* q, const float* k, const float* v,
                           const float* alpha, const float* beta, const float* o) {
  if (!q || !k || !v || !alpha || !beta || !o)
    return fail(LSQ_ERR_INVALID_ARG, "q, k, v, alpha, beta and o must be non-null");
  if (!aligned16(q) || !aligned16(k) || (st->cfg.decay == LSQ_DECAY_DIAG && !aligned16(alpha)))
    return fail(LSQ_ERR_INVALID_ARG, "q, k (and a diagonal alpha) must be 16-byte aligned");
  if (!aligned4(v) || !aligned4(alpha) || !aligned4(beta) || !aligned4(o))
    return fail(LSQ_ERR_INVALID_ARG, "v, alpha, beta and o must be 4-byte aligned");
  return ok();
}

lsq_status launch_one_step(lsq_state* st, const float* q, const float* k, const float* v,
                           const float* alpha, const float* beta, float* o, float* o_ref,
                           hipStream_t stream) {
  const lsq_config& c = st->cfg;
  if (n_heads(c) == 0) return ok();
  lsq::StepArgs a{};
  a.codes = static_cast<uint8_t*>(st->codes);
  a.scales = st->scales;
  a.sfmt = st->cfg.scale_fmt;
  a.ref = (c.bits == 32) ? st->f32 : st->ref;
  a.q = q; a.k = k; a.v = v; a.alpha = alpha; a.beta = beta; a.o = o;
  a.o_ref = (c.policy == LSQ_POLICY_YOKED) ? o_ref : nullptr;
  a.n_heads = (int32_t)n_heads(c);
  a.dv = c.dv;
  a.group = c.group;
  a.ng = (c.bits == 32 || c.group == 0) ? 0 : c.dk / c.group;
  if (c.bits != 32 && c.group == 0 && c.policy == LSQ_POLICY_PERSISTENT) {
    // a frozen head scale: the main step kernel with row groups of Dk whose
    // scale address does not move with the row
    a.group = c.dk;
    a.head_scale = 1;
  }
  // The plain quantised step (no bypass buffer, no fp32 reference) on a state
  // of few heads: each wave stages its head's vectors before its first row, so
  // fewer, longer waves (4096: four per SIMD, each with the next row in flight)
  // pay that set-up less often.  Measured on 1024 heads with a diagonal decay
  // (median launch): 13.6 us at 1024 waves, 10.9 at 2048, 10.4 at 4096, 10.5 at
  // 8192 and 16384; 4096 dynamic-scale heads and 8192 Mamba-2-style heads are
  // within 2% from 1024 to 8192 waves; a state of more heads than that already
  // runs one wave per head either way.
  const bool lean = c.bits != 32 && c.lrb_rank == 0 && c.policy != LSQ_POLICY_YOKED &&
                    c.rounding != LSQ_ROUND_BDR_A && c.rounding != LSQ_ROUND_BDR_B &&
                    !(c.group == 0 && c.policy == LSQ_POLICY_DYNAMIC);
  choose_slices(c, &a.nit, &a.waves_per_head, &a.total_waves, lean ? LSQ_LEAN_WAVES : 8192);
  // a state of 512 MiB or more does not stay in the 256 MB Infinity Cache
  // between steps: its code loads take the non-temporal hint
  a.nt_loads = (size_t)n_heads(c) * c.dv * c.dk * (size_t)c.bits / 8 >= ((size_t)512 << 20);
  constexpr uint32_t kWeyl = 0x9E3779B9u;   // 2^32 (sqrt(5)-1)/2, truncated
  a.dither_base = (uint32_t)((uint64_t)st->step * (uint64_t)c.dv * (uint64_t)c.dk) * kWeyl;
  a.dither_row = (uint32_t)c.dk * kWeyl;
  hipError_t e;
  if (c.lrb_rank > 0) {
    const int64_t r = c.lrb_rank;
    a.lrb_a = st->lrb;
    a.lrb_b = st->lrb + n_heads(c) * r * c.dv;
    a.lrb_rank = c.lrb_rank;
    a.lrb_used = (int32_t)(st->step % r);
    a.lrb_merge = a.lrb_used == c.lrb_rank - 1;
    a.lrb_cin = (c.decay == LSQ_DECAY_DIAG) ? (int32_t)(st->step & 1) : 0;
    a.lrb_cout = (c.decay == LSQ_DECAY_DIAG) ? (int32_t)((st->step + 1) & 1) : 0;
    e = lsq::launch_lrb_step(a, c.bits, c.dk, c.policy, c.rounding, c.delta, c.decay, stream);
  } else if (c.bits == 32)
    e = lsq::launch_step_f32(a, c.dk, c.delta, c.decay, stream);
  else if (c.group == 0 && c.policy == LSQ_POLICY_DYNAMIC)
    e = lsq::launch_head_scale(a, c.bits, c.dk, c.policy, c.rounding, c.delta, c.decay, stream);
  else if (c.rounding == LSQ_ROUND_BDR_A || c.rounding == LSQ_ROUND_BDR_B)
    e = lsq::launch_bdr_alt(a, c.bits, c.dk, c.rounding, c.delta, c.decay, stream);
  else if (c.scale_fmt != LSQ_SCALE_F32)
    e = (c.bits == 4 ? (c.scale_fmt == LSQ_SCALE_F16 ? lsq::launch_step_q4_f16 : lsq::launch_step_q4_bf16)
                     : (c.scale_fmt == LSQ_SCALE_F16 ? lsq::launch_step_q8_f16 : lsq::launch_step_q8_bf16))(
        a, c.dk, c.policy, c.rounding, c.delta, c.decay, stream);
  else if (c.bits == 4)
    e = lsq::launch_step_q4(a, c.dk, c.policy, c.rounding, c.delta, c.decay, stream);
  else
    e = lsq::launch_step_q8(a, c.dk, c.policy, c.rounding, c.delta, c.decay, stream);
  lsq_status s = hip_status(e, "decode-step launch");
  if (s == LSQ_OK) ++st->step;
  return s;
}

}  // namespace

extern "C" {

lsq_status lsq_state_sizes(const lsq_config* cfg, size_t* codes_bytes, size_t* scales_bytes,
                           size_t* ref_bytes, size_t* f32_bytes, size_t* lrb_bytes) {
  lsq_status s = check_config(cfg);
  if (s != LSQ_OK) return s;
  size_t sz[kBuffers];
  sizes_of(*cfg, sz);
  size_t* out[kBuffers] = {codes_bytes, scales_bytes, ref_bytes, f32_bytes, lrb_bytes};
  for (int i = 0; i < kBuffers; ++i)
    if (out[i]) *out[i] = sz[i];
  return ok();
}

lsq_status lsq_state_alloc(const lsq_config* cfg, const lsq_buffers* bufs, lsq_state** out) {
  if (!out) return fail(LSQ_ERR_INVALID_ARG, "out is null");
  *out = nullptr;
  lsq_status s = check_config(cfg);
  if (s != LSQ_OK) return s;
  if (!bufs) return fail(LSQ_ERR_INVALID_ARG, "buffers are null");
  size_t need[kBuffers];
  sizes_of(*cfg, need);
  const void* ptr[kBuffers] = {bufs->codes, bufs->scales, bufs->ref, bufs->f32, bufs->lrb};
  const size_t cap[kBuffers] = {bufs->codes_bytes, bufs->scales_bytes, bufs->ref_bytes,
                                bufs->f32_bytes, bufs->lrb_bytes};
  static const char* names[kBuffers] = {"codes", "scales", "ref", "f32", "lrb"};
  for (int i = 0; i < kBuffers; ++i) {
    if (need[i] == 0) continue;
    if (!ptr[i]) return fail(LSQ_ERR_INVALID_ARG, "%s buffer is null", names[i]);
    if (!aligned16(ptr[i])) return fail(LSQ_ERR_INVALID_ARG, "%s buffer is not 16-byte aligned", names[i]);
    if (cap[i] < need[i])
      return fail(LSQ_ERR_BUFFER_TOO_SMALL, "%s buffer holds %zu bytes, needs %zu", names[i],
                  cap[i], need[i]);
  }
  lsq_state* st = new (std::nothrow) lsq_state;
  if (!st) return fail(LSQ_ERR_INVALID_ARG, "host allocation of the handle failed");
  st->cfg = *cfg;
  st->codes = need[0] ? bufs->codes : nullptr;
  st->scales = need[1] ? bufs->scales : nullptr;
  st->ref = need[2] ? bufs->ref : nullptr;
  st->f32 = need[3] ? bufs->f32 : nullptr;
  st->lrb = need[4] ? bufs->lrb : nullptr;
  st->calibrated = 0;
  st->step = 0;
  *out = st;
  return ok();
}

void lsq_state_free(lsq_state* st) { delete st; }

lsq_status lsq_state_config(const lsq_state* st, lsq_config* out) {
  if (!st || !out) return fail(LSQ_ERR_INVALID_ARG, "null argument");
  *out = st->cfg;
  return ok();
}

lsq_status lsq_state_zero(lsq_state* st, void* stream) {
  if (!st) return fail(LSQ_ERR_INVALID_ARG, "state is null");
  size_t need[kBuffers];
  sizes_of(st->cfg, need);
  void* ptr[kBuffers] = {st->codes, st->scales, st->ref, st->f32, st->lrb};
  hipStream_t hs = static_cast<hipStream_t>(stream);
  for (int i = 0; i < kBuffers; ++i) {
    if (!need[i]) continue;
    lsq_status s = hip_status(lsq::launch_fill_zero(ptr[i], need[i], hs), "zero fill");
    if (s != LSQ_OK) return s;
  }
  st->calibrated = 0;
  st->step = 0;
  return ok();
}

lsq_status lsq_state_dequantize(const lsq_state* st, float* S, void* stream) {
  if (!st) return fail(LSQ_ERR_INVALID_ARG, "state is null");
  const lsq_config& c = st->cfg;
  hipStream_t hs = static_cast<hipStream_t>(stream);
  const size_t elems = (size_t)n_heads(c) * c.dv * c.dk;
  if (elems == 0) return ok();
  if (!S) return fail(LSQ_ERR_INVALID_ARG, "S is null");
  if (!aligned16(S)) return fail(LSQ_ERR_INVALID_ARG, "S must be 16-byte aligned");
  if (c.bits == 32)                    // the state is already fp32
    return hip_status(hipMemcpyAsync(S, st->f32, elems * 4, hipMemcpyDeviceToDevice, hs),
                      "dequantize copy");
  lsq::DequantArgs a{};
  a.codes = static_cast<const uint8_t*>(st->codes);
  a.scales = st->scales;
  a.S = S;
  a.rows = (int64_t)n_heads(c) * c.dv;
  a.dv = c.dv;
  a.group = c.group;
  a.ng = c.group ? c.dk / c.group : 0;
  a.sfmt = c.scale_fmt;
  return hip_status(lsq::launch_dequantize(a, c.bits, c.dk, hs), "dequantize launch");
}

lsq_status lsq_state_calibrate(lsq_state* st, const float* S, void* stream) {
  if (!st) return fail(LSQ_ERR_INVALID_ARG, "state is null");
  const lsq_config& c = st->cfg;
  hipStream_t hs = static_cast<hipStream_t>(stream);
  const size_t elems = (size_t)n_heads(c) * c.dv * c.dk;
  if (elems == 0) {   // nothing to read or write
    st->calibrated = 1;
    return ok();
  }
  if (!S) return fail(LSQ_ERR_INVALID_ARG, "S is null");
  if (!aligned16(S)) return fail(LSQ_ERR_INVALID_ARG, "S must be 16-byte aligned");
  if (c.bits == 32) {
    lsq_status s = hip_status(hipMemcpyAsync(st->f32, S, elems * 4, hipMemcpyDeviceToDevice, hs),
                              "calibrate copy");
    if (s == LSQ_OK) st->calibrated = 1;
    return s;
  }
  lsq::CalibArgs a{};
  a.S = S;
  a.codes = static_cast<uint8_t*>(st->codes);
  a.scales = st->scales;
  a.sfmt = st->cfg.scale_fmt;
  a.ref = (c.policy == LSQ_POLICY_YOKED) ? st->ref : nullptr;
  a.n_heads = (int32_t)n_heads(c);
  a.dv = c.dv;
  a.group = c.group;
  if (c.group == 0) {                  // one scale per head
    a.ng = 0;
    lsq_status s = hip_status(lsq::launch_calibrate_head(a, c.bits, c.dk, hs), "calibrate launch");
    if (s == LSQ_OK) st->calibrated = 1;
    return s;
  }
  a.ng = c.dk / c.group;
  choose_slices(c, &a.nit, &a.waves_per_head, &a.total_waves);
  lsq_status s = hip_status(lsq::launch_calibrate(a, c.bits, c.dk, hs), "calibrate launch");
  if (s == LSQ_OK) st->calibrated = 1;
  return s;
}

lsq_status lsq_state_set_calibrated(lsq_state* st, int32_t calibrated) {
  if (!st) return fail(LSQ_ERR_INVALID_ARG, "state is null");
  st->calibrated = calibrated ? 1 : 0;
  return ok();
}

lsq_status lsq_state_step_index(const lsq_state* st, int64_t* out) {
  if (!st || !out) return fail(LSQ_ERR_INVALID_ARG, "null argument");
  *out = st->step;
  return ok();
}

lsq_status lsq_state_set_step_index(lsq_state* st, int64_t step) {
  if (!st) return fail(LSQ_ERR_INVALID_ARG, "state is null");
  if (step < 0) return fail(LSQ_ERR_INVALID_ARG, "negative step index");
  st->step = step;
  return ok();
}

lsq_status lsq_decode_step(lsq_state* st, const float* q, const float* k, const float* v,
                           const float* alpha, const float* beta, float* o, float* o_ref,
                           void* stream) {
  if (!st) return fail(LSQ_ERR_INVALID_ARG, "state is null");
  if (st->cfg.policy == LSQ_POLICY_PERSISTENT && !st->calibrated)
    return fail(LSQ_ERR_NOT_CALIBRATED, "persistent scale used before lsq_state_calibrate");
  if (n_heads(st->cfg) == 0) {   // nothing to read or write
    ++st->step;
    return ok();
  }
  lsq_status s = check_step_ptrs(st, q, k, v, alpha, beta, o);
  if (s != LSQ_OK) return s;
  return launch_one_step(st, q, k, v, alpha, beta, o, o_ref, static_cast<hipStream_t>(stream));
}

lsq_status lsq_decode_run(lsq_state* st, int32_t H, const float* q, const float* k,
                          const float* v, const float* alpha, const float* beta, float* o,
                          float* o_ref, void* stream) {
  if (!st) return fail(LSQ_ERR_INVALID_ARG, "state is null");
  if (H < 0) return fail(LSQ_ERR_INVALID_ARG, "negative horizon");
  if (st->cfg.policy == LSQ_POLICY_PERSISTENT && !st->calibrated)
    return fail(LSQ_ERR_NOT_CALIBRATED, "persistent scale used before lsq_state_calibrate");
  if (H == 0 || n_heads(st->cfg) == 0) {   // nothing to read or write
    st->step += H;
    return ok();
  }
  lsq_status s = check_step_ptrs(st, q, k, v, alpha, beta, o);
  if (s != LSQ_OK) return s;
  const lsq_config& c = st->cfg;
  const size_t n = (size_t)n_heads(c);
  const size_t sq = n * c.dk, sv = n * c.dv;
  const size_t sa = (c.decay == LSQ_DECAY_DIAG) ? n * c.dk : n;
  hipStream_t hs = static_cast<hipStream_t>(stream);
  for (int32_t t = 0; t < H; ++t) {
    s = launch_one_step(st, q + t * sq, k + t * sq, v + t * sv, alpha + t * sa, beta + t * n,
                        o + t * sv, o_ref ? o_ref + t * sv : nullptr, hs);
    if (s != LSQ_OK) return s;
  }
  return ok();
}

lsq_status lsq_prefill(lsq_state* st, int32_t T, const float* k, const float* v,
                       const float* alpha, const float* beta, void* stream) {
  if (!st) return fail(LSQ_ERR_INVALID_ARG, "state is null");
  if (T < 0) return fail(LSQ_ERR_INVALID_ARG, "negative token count");
  const lsq_config& c = st->cfg;
  if (c.bits != 4 && c.bits != 8) return fail(LSQ_ERR_UNSUPPORTED, "prefill needs a quantised state");
  if (c.policy != LSQ_POLICY_DYNAMIC && c.policy != LSQ_POLICY_PERSISTENT)
    return fail(LSQ_ERR_UNSUPPORTED, "prefill supports the DYNAMIC and PERSISTENT policies");
  if (c.delta != 0) return fail(LSQ_ERR_UNSUPPORTED, "prefill supports the linear write (delta 0)");
  if (c.lrb_rank != 0) return fail(LSQ_ERR_UNSUPPORTED, "prefill does not take the bypass");
  if (c.dv != 64 && c.dv != 128)
    return fail(LSQ_ERR_UNSUPPORTED, "dv %d: prefill has dv 64 and 128", c.dv);
  if (c.group != 0 && c.dk / c.group > 8)
    return fail(LSQ_ERR_UNSUPPORTED, "prefill holds at most 8 groups per row");
  if (c.policy == LSQ_POLICY_PERSISTENT && !st->calibrated)
    return fail(LSQ_ERR_NOT_CALIBRATED, "persistent scale used before lsq_state_calibrate");
  if (T == 0 || n_heads(c) == 0) {
    st->step += T;
    return ok();
  }
  if (!k || !v || !alpha || !beta) return fail(LSQ_ERR_INVALID_ARG, "k, v, alpha and beta must be non-null");
  if (!aligned4(k) || !aligned4(v) || !aligned4(alpha) || !aligned4(beta))
    return fail(LSQ_ERR_INVALID_ARG, "k, v, alpha and beta must be 4-byte aligned");
  if (n_heads(c) > INT32_MAX) return fail(LSQ_ERR_UNSUPPORTED, "too many heads for one launch");
  lsq::PrefillArgs a{};
  a.codes = static_cast<uint8_t*>(st->codes);
  a.scales = st->scales;
  a.k = k;
  a.v = v;
  a.alpha = alpha;
  a.beta = beta;
  a.n_heads = (int32_t)n_heads(c);
  a.T = T;
  a.ng = c.group ? c.dk / c.group : 0;       // group 0: one scale per head
  a.group = c.group;
  a.sfmt = c.scale_fmt;
  hipError_t e = lsq::launch_prefill(a, c.bits, c.dk, c.dv, c.policy,
                                     c.decay == LSQ_DECAY_DIAG, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_status(e, "prefill launch");
  st->step += T;
  return ok();
}

lsq_status lsq_probe_stream(int32_t kind, const void* src, void* dst, size_t bytes,
                            int32_t loads_per_lane, int32_t nontemporal, int32_t workgroups,
                            void* stream) {
  if (kind != LSQ_PROBE_READ && kind != LSQ_PROBE_WRITE && kind != LSQ_PROBE_COPY)
    return fail(LSQ_ERR_INVALID_ARG, "probe kind must be READ, WRITE or COPY");
  if (bytes % 16 != 0) return fail(LSQ_ERR_INVALID_ARG, "probe size must be a multiple of 16 bytes");
  if (loads_per_lane != 1 && loads_per_lane != 2 && loads_per_lane != 4 && loads_per_lane != 8)
    return fail(LSQ_ERR_INVALID_ARG, "loads_per_lane must be 1, 2, 4 or 8");
  if (nontemporal != 0 && nontemporal != 1)
    return fail(LSQ_ERR_INVALID_ARG, "nontemporal must be 0 or 1");
  if (workgroups < 0) return fail(LSQ_ERR_INVALID_ARG, "negative workgroup count");
  if (bytes == 0) return ok();
  if (kind != LSQ_PROBE_WRITE && (!src || !aligned16(src)))
    return fail(LSQ_ERR_INVALID_ARG, "probe source must be non-null and 16-byte aligned");
  if (!dst || !aligned16(dst))
    return fail(LSQ_ERR_INVALID_ARG, "probe destination must be non-null and 16-byte aligned");
  const size_t tile = (size_t)256 * loads_per_lane * 16;
  if (workgroups == 0 && (bytes + tile - 1) / tile > (size_t)INT32_MAX)
    return fail(LSQ_ERR_UNSUPPORTED, "probe size too large for a single pass");
  hipError_t e = lsq::launch_probe(kind, src, dst, bytes, loads_per_lane, nontemporal, workgroups,
                                   static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_status(e, "probe launch");
  return ok();
}

lsq_status lsq_probe_span(const void* src, void* dst, size_t bytes, int32_t span_kib,
                          int32_t nontemporal, void* stream) {
  if (span_kib != 1 && span_kib != 2 && span_kib != 4 && span_kib != 8 && span_kib != 10 &&
      span_kib != 16)
    return fail(LSQ_ERR_INVALID_ARG, "span_kib must be 1, 2, 4, 8, 10 or 16");
  if (nontemporal != 0 && nontemporal != 1)
    return fail(LSQ_ERR_INVALID_ARG, "nontemporal must be 0 or 1");
  if (bytes % ((size_t)span_kib * 1024) != 0)
    return fail(LSQ_ERR_INVALID_ARG, "probe size must be a multiple of the span");
  if (bytes / ((size_t)span_kib * 1024) > (size_t)INT32_MAX / 4)
    return fail(LSQ_ERR_UNSUPPORTED, "probe size too large for one launch");
  if (bytes == 0) return ok();
  if (!src || !dst || !aligned16(src) || !aligned16(dst))
    return fail(LSQ_ERR_INVALID_ARG, "probe buffers must be non-null and 16-byte aligned");
  hipError_t e = lsq::launch_probe_span(src, dst, bytes, span_kib, nontemporal,
                                        static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_status(e, "probe launch");
  return ok();
}

lsq_status lsq_probe_valu(int32_t form, int32_t workgroups, int32_t iters, float* out,
                          void* stream) {
  if (form < LSQ_PROBE_VALU_FMA || form > LSQ_PROBE_VALU_MUL)
    return fail(LSQ_ERR_INVALID_ARG, "VALU probe form must be one of lsq_probe_valu_form (0-9)");
  if (workgroups < 1 || iters < 1)
    return fail(LSQ_ERR_INVALID_ARG, "VALU probe needs at least one workgroup and one iteration");
  if (!out) return fail(LSQ_ERR_INVALID_ARG, "VALU probe output must be non-null");
  hipError_t e = lsq::launch_probe_valu(form, workgroups, iters, out, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_status(e, "probe launch");
  return ok();
}

const char* lsq_status_string(lsq_status s) {
  switch (s) {
    case LSQ_OK: return "LSQ_OK";
    case LSQ_ERR_INVALID_ARG: return "LSQ_ERR_INVALID_ARG: invalid argument";
    case LSQ_ERR_UNSUPPORTED: return "LSQ_ERR_UNSUPPORTED: configuration not supported by this library";
    case LSQ_ERR_BUFFER_TOO_SMALL: return "LSQ_ERR_BUFFER_TOO_SMALL: a state buffer is too small";
    case LSQ_ERR_NOT_CALIBRATED: return "LSQ_ERR_NOT_CALIBRATED: persistent scales not calibrated";
    case LSQ_ERR_HIP: return "LSQ_ERR_HIP: HIP runtime error";
  }
  return "unknown lsq_status";
}

const char* lsq_last_error(void) { return g_last_error.c_str(); }

int32_t lsq_version(void) { return 103; }

}  // extern "C"
