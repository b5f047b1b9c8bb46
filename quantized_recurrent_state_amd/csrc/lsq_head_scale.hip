// Decode step and calibration with one scale per head (group = 0): the
// coarsest scale granularity, one fp32 scale for a head's whole Dv x Dk state.
//
// The scale-format variants of "Preserving Updates in Low-Bit Recurrent State
// Quantization" (its memory figure leaves the format open) and the per-token
// dynamic scale of "When Dynamic Scaling Fails" (project page, mechanism
// paragraph) at head granularity.  A dynamic per-head scale depends on every
// row's update, so no row can be requantised before all rows are updated.
// Heads of at most sixteen row-iterations take head_scale1_kernel (below):
// one row-iteration per wave of an eight- or sixteen-wave workgroup, every
// row held in registers across the barrier.  Taller heads take this kernel: one
// workgroup (four waves) per head makes two passes over the head's rows.
//   pass 1  per row: codes -> S' = fl(C fl(s alpha)), u = S'.k, w = beta (v -
//           delta u), S = fma(w, k, S'), o = S.q (written); the row's w kept
//           in LDS; the lanes' running max |S|;
//   scale   workgroup max -> s_new = fl(max/qmax) (dynamic) or s (persistent),
//           inv = fl(1/s_new);
//   pass 2  per row again (codes re-read, mostly from L2): the same S' and S,
//           then round half to even, or directional rounding (sigma =
//           sign(w) sign(k_c); a code c1 with (c1 - S' inv) sigma < 0, decided
//           exactly by the sign of one fma, becomes c1 + sigma, clamped).
// A persistent (frozen) head scale is known in advance, so that policy runs in
// the main step kernel with the head's scale broadcast to every row; this
// kernel holds the dynamic policy.
// Lane layout as the main step: 32 consecutive elements of a row per lane.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "lsq_step_impl.h"

namespace lsq {
namespace dev {

constexpr int kHeadWaves = 4;
constexpr int kMaxDv = 1024;           // LDS rows of w (the host checks dv)

__device__ __forceinline__ float wave_max_all(float x) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x = fmaxf(x, __shfl_xor(x, o));
  return x;
}

template <int BITS, int DK, int POLICY, int ROUND, int DELTA, int DIAG>
__global__ __launch_bounds__(256) void head_scale_kernel(StepArgs a) {
  static_assert(POLICY == POL_DYNAMIC, "a frozen head scale runs in the main step kernel");
  using F = Fmt<BITS>;
  constexpr int NW = F::NW, LPR = DK / EPL, RPI = 64 / LPR, ROWB = DK * BITS / 8;
  constexpr bool BDR = ROUND == RND_BDR;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int h = blockIdx.x;
  const int lr = lane / LPR, lc = lane % LPR, col0 = lc * EPL;
  __shared__ float wrow[kMaxDv];
  __shared__ float wmax[kHeadWaves];

  float kk[EPL], qq[EPL], al[DIAG ? EPL : 4];
  load_f32(kk, a.k + (size_t)h * DK + col0);
  load_f32(qq, a.q + (size_t)h * DK + col0);
  if constexpr (DIAG) load_f32(al, a.alpha + (size_t)h * DK + col0);
  else al[0] = a.alpha[h];
  const float beta = a.beta[h];
  const float s = a.scales[h];
  float m[DIAG ? EPL : 1];
#pragma unroll
  for (int e = 0; e < (DIAG ? EPL : 1); ++e) m[e] = s * al[e];
  const int iters = (a.dv + kHeadWaves * RPI - 1) / (kHeadWaves * RPI);

  // S' and S of one row from its codes (identical in both passes)
  auto update = [&](size_t row, float w_in, bool have_w, float (&sp)[EPL], float (&st)[EPL],
                    float& w_out) {
    const uint8_t* cp = a.codes + row * ROWB + lc * (EPL * BITS / 8);
    uint32_t xo[NW];
#pragma unroll
    for (int c = 0; c < NW / 4; ++c) {
      const u32x4 w4 = load_codes16<>(cp + 16 * c);
      xo[4 * c + 0] = w4.x ^ F::OFF;
      xo[4 * c + 1] = w4.y ^ F::OFF;
      xo[4 * c + 2] = w4.z ^ F::OFF;
      xo[4 * c + 3] = w4.w ^ F::OFF;
    }
    float cu[EPL];
    unpack_offsets<BITS>(xo, cu);
    float pu = 0.f;
#pragma unroll
    for (int e = 0; e < EPL; ++e) {
      sp[e] = (cu[e] - F::BIAS) * m[DIAG ? e : 0];
      if constexpr (DELTA) pu = fmaf(sp[e], kk[e], pu);
    }
    float w = w_in;
    if (!have_w) {
      const float u = DELTA ? row_sum<LPR>(pu) : 0.f;
      w = beta * (a.v[row] - u);
    }
#pragma unroll
    for (int e = 0; e < EPL; ++e) st[e] = fmaf(w, kk[e], sp[e]);
    w_out = w;
  };

  // requantise one row with the head's inverse scale and store its codes
  auto requant_store = [&](size_t row, bool live, float w, const float (&sp)[EPL],
                           const float (&st)[EPL], float inv) {
    const int sw = (w > 0.f) - (w < 0.f);
    float t[EPL];
#pragma unroll
    for (int e = 0; e < EPL; ++e) {
      t[e] = __builtin_amdgcn_fmed3f(fmaf(st[e], inv, F::MQ), F::MQ - F::QMAX, F::MQ + F::QMAX);
      if constexpr (BDR) {
        const int sigma = sw * ((kk[e] > 0.f) - (kk[e] < 0.f));
        const float d = fmaf(sp[e], inv, F::MQ - t[e]);     // S' inv - c1, one rounding
        const bool rev = (sigma > 0 && d > 0.f) || (sigma < 0 && d < 0.f);
        if (rev)
          t[e] = __builtin_amdgcn_fmed3f(t[e] + (float)sigma, F::MQ - F::QMAX, F::MQ + F::QMAX);
      }
    }
    uint32_t X[NW];
    pack_offsets<BITS>(t, X);
    if (live) {
      uint8_t* cp = a.codes + row * ROWB + lc * (EPL * BITS / 8);
#pragma unroll
      for (int c = 0; c < NW / 4; ++c)
        store_codes16(cp + 16 * c, u32x4{X[4 * c] ^ F::OFF, X[4 * c + 1] ^ F::OFF,
                                         X[4 * c + 2] ^ F::OFF, X[4 * c + 3] ^ F::OFF});
    }
  };
  // ---- pass 1: update every row, outputs, w, running max
  float amax = 0.f;
  for (int it = 0; it < iters; ++it) {
    const int r = (it * kHeadWaves + wave) * RPI + lr;
    const bool live = r < a.dv;
    const size_t row = (size_t)h * a.dv + (live ? r : a.dv - 1);
    float sp[EPL], st[EPL], w;
    update(row, 0.f, false, sp, st, w);
    float po = 0.f;
#pragma unroll
    for (int e = 0; e < EPL; ++e) {
      po = fmaf(st[e], qq[e], po);
      if (live) amax = fmaxf(amax, fabsf(st[e]));
    }
    const float o = row_sum<LPR>(po);
    if (live && lc == 0) {
      a.o[row] = o;
      wrow[r] = w;
    }
  }
  float snew = s;
  if constexpr (POLICY == POL_DYNAMIC) {
    amax = wave_max_all(amax);
    if (lane == 0) wmax[wave] = amax;
  }
  __syncthreads();
  if constexpr (POLICY == POL_DYNAMIC) {
    float mx = wmax[0];
#pragma unroll
    for (int i = 1; i < kHeadWaves; ++i) mx = fmaxf(mx, wmax[i]);
    snew = mx / F::QMAX;
  }
  const float inv = inv_scale(snew);

  // ---- pass 2: the same updates, requantised with the head's scale
  for (int it = 0; it < iters; ++it) {
    const int r = (it * kHeadWaves + wave) * RPI + lr;
    const bool live = r < a.dv;
    const size_t row = (size_t)h * a.dv + (live ? r : a.dv - 1);
    float sp[EPL], st[EPL], w;
    update(row, wrow[live ? r : a.dv - 1], true, sp, st, w);
    requant_store(row, live, w, sp, st, inv);
  }
  if constexpr (POLICY == POL_DYNAMIC) {
    if (tid == 0) a.scales[h] = snew;
  }
}

// The same step for heads of at most NWV x (rows per wave-iteration) rows
// (NWV = 8: 128 rows at Dk = 128; NWV = 16: 256): one workgroup of NWV waves
// per head, one row-iteration per wave, so every row's S' and S stay in
// registers across the workgroup barrier and the codes are read once.  k, q and a diagonal decay are staged
// in LDS.  Pass 1 (update, o, running max) and pass 2 (requantisation) are
// the two halves of the same per-row computation as above; the values, the
// rounding and the stored results are the same.
template <int BITS, int DK, int ROUND, int DELTA, int DIAG, int NWV>
__global__ __launch_bounds__(64 * NWV) void head_scale1_kernel(StepArgs a) {
  using F = Fmt<BITS>;
  constexpr int NW = F::NW, LPR = DK / EPL, RPI = 64 / LPR, ROWB = DK * BITS / 8;
  constexpr bool BDR = ROUND == RND_BDR;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int h = blockIdx.x;
  const int lr = lane / LPR, lc = lane % LPR, col0 = lc * EPL;
  __shared__ float4 vec4[(DIAG ? 3 : 2) * DK / 4];
  __shared__ float wmax[NWV];
  float* kv = reinterpret_cast<float*>(vec4);
  float* qv = kv + DK;
  float* av = kv + 2 * DK;

  // this lane's row: its codes and v are requested before the vectors are staged
  const int r = wave * RPI + lr;
  const bool live = r < a.dv;
  const uint32_t i = (uint32_t)(live ? r : a.dv - 1);
  uint8_t* const codes_h = a.codes + (size_t)h * a.dv * ROWB;
  uint32_t xo[NW];
#pragma unroll
  for (int c = 0; c < NW / 4; ++c) {
    const u32x4 w4 = load_codes16<>(codes_h + (i * ROWB + lc * (EPL * BITS / 8) + 16 * c));
    xo[4 * c + 0] = w4.x ^ F::OFF;
    xo[4 * c + 1] = w4.y ^ F::OFF;
    xo[4 * c + 2] = w4.z ^ F::OFF;
    xo[4 * c + 3] = w4.w ^ F::OFF;
  }
  const float vr = a.v[(size_t)h * a.dv + i];
  const float s = a.scales[h];
  const float beta = a.beta[h];
  const float alpha_s = DIAG ? 1.f : a.alpha[h];
  if (tid < DK) {
    kv[tid] = a.k[(size_t)h * DK + tid];
    qv[tid] = a.q[(size_t)h * DK + tid];
    if constexpr (DIAG) av[tid] = a.alpha[(size_t)h * DK + tid];
  }
  __syncthreads();

  // pass 1: S' = fl(C fl(s alpha)), u, w, S = fma(w, k, S'), o, max |S|
  float sp[EPL];
  if constexpr (DIAG) {
    unpack_offsets<BITS>(xo, sp);
#pragma unroll
    for (int b = 0; b < EPL / 8; ++b) {
      float ab[8];
      lds_block<DK>(ab, av, col0 + 8 * b);
#pragma unroll
      for (int e8 = 0; e8 < 8; ++e8) sp[8 * b + e8] = (sp[8 * b + e8] - F::BIAS) * (s * ab[e8]);
    }
  } else {
    const float m[1] = {s * alpha_s}, mb[1] = {-F::BIAS * (s * alpha_s)};
    dequant_mix<BITS, 1>(xo, m, mb, sp);
  }
  float u = 0.f;
  if constexpr (DELTA) {
    float pu = 0.f;
#pragma unroll
    for (int b = 0; b < EPL / 8; ++b) {
      float kb[8];
      lds_block<DK>(kb, kv, col0 + 8 * b);
#pragma unroll
      for (int e8 = 0; e8 < 8; ++e8) pu = fmaf(sp[8 * b + e8], kb[e8], pu);
    }
    u = row_sum<LPR>(pu);
  }
  const float w = beta * (vr - u);
  float st[EPL];
  float po = 0.f, amax = 0.f;
#pragma unroll
  for (int b = 0; b < EPL / 8; ++b) {
    float kb[8], qb[8];
    lds_block<DK>(kb, kv, col0 + 8 * b);
    lds_block<DK>(qb, qv, col0 + 8 * b);
#pragma unroll
    for (int e8 = 0; e8 < 8; ++e8) {
      st[8 * b + e8] = fmaf(w, kb[e8], sp[8 * b + e8]);
      po = fmaf(st[8 * b + e8], qb[e8], po);
      amax = fmaxf(amax, fabsf(st[8 * b + e8]));
    }
  }
  const float o = row_sum<LPR>(po);
  if (live && lc == 0) a.o[(size_t)h * a.dv + i] = o;
  if (!live) amax = 0.f;
  amax = wave_max_all(amax);
  if (lane == 0) wmax[wave] = amax;
  __syncthreads();
  float mx = wmax[0];
#pragma unroll
  for (int j = 1; j < NWV; ++j) mx = fmaxf(mx, wmax[j]);
  const float snew = mx / F::QMAX;
  const float inv = inv_scale(snew);

  // pass 2: round half to even, or directional rounding (sigma = sign(w) sign(k_c);
  // a code c1 with (c1 - S' inv) sigma < 0, decided by the sign of one fma,
  // becomes c1 + sigma, clamped)
  const int sw = (w > 0.f) - (w < 0.f);
  float t[EPL];
#pragma unroll
  for (int b = 0; b < EPL / 8; ++b) {
    float kb[8];
    if constexpr (BDR) lds_block<DK>(kb, kv, col0 + 8 * b);
#pragma unroll
    for (int e8 = 0; e8 < 8; ++e8) {
      const int e = 8 * b + e8;
      t[e] = __builtin_amdgcn_fmed3f(fmaf(st[e], inv, F::MQ), F::MQ - F::QMAX, F::MQ + F::QMAX);
      if constexpr (BDR) {
        const int sigma = sw * ((kb[e8] > 0.f) - (kb[e8] < 0.f));
        const float d = fmaf(sp[e], inv, F::MQ - t[e]);     // S' inv - c1, one rounding
        const bool rev = (sigma > 0 && d > 0.f) || (sigma < 0 && d < 0.f);
        const float step = rev ? (float)sigma : 0.f;
        t[e] = __builtin_amdgcn_fmed3f(t[e] + step, F::MQ - F::QMAX, F::MQ + F::QMAX);
      }
    }
  }
  uint32_t X[NW];
  pack_offsets<BITS>(t, X);
  if (live) {
#pragma unroll
    for (int c = 0; c < NW / 4; ++c)
      store_codes16(codes_h + (i * ROWB + lc * (EPL * BITS / 8) + 16 * c),
                    u32x4{X[4 * c] ^ F::OFF, X[4 * c + 1] ^ F::OFF, X[4 * c + 2] ^ F::OFF,
                          X[4 * c + 3] ^ F::OFF});
  }
  if (tid == 0) a.scales[h] = snew;
}

// Calibration with one scale per head: absmax over the head, then RNE codes.
template <int BITS, int DK>
__global__ __launch_bounds__(256) void calibrate_head_kernel(CalibArgs a) {
  using F = Fmt<BITS>;
  constexpr int NW = F::NW, LPR = DK / EPL, RPI = 64 / LPR, ROWB = DK * BITS / 8;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int h = blockIdx.x;
  const int lr = lane / LPR, lc = lane % LPR, col0 = lc * EPL;
  __shared__ float wmax[kHeadWaves];
  const int iters = (a.dv + kHeadWaves * RPI - 1) / (kHeadWaves * RPI);
  float amax = 0.f;
  for (int it = 0; it < iters; ++it) {
    const int r = (it * kHeadWaves + wave) * RPI + lr;
    if (r >= a.dv) continue;
    float x[EPL];
    load_f32(x, a.S + ((size_t)h * a.dv + r) * DK + col0);
#pragma unroll
    for (int e = 0; e < EPL; ++e) amax = fmaxf(amax, fabsf(x[e]));
  }
  amax = wave_max_all(amax);
  if (lane == 0) wmax[wave] = amax;
  __syncthreads();
  float mx = wmax[0];
#pragma unroll
  for (int i = 1; i < kHeadWaves; ++i) mx = fmaxf(mx, wmax[i]);
  const float s = mx / F::QMAX;
  const float inv = inv_scale(s);
  for (int it = 0; it < iters; ++it) {
    const int r = (it * kHeadWaves + wave) * RPI + lr;
    if (r >= a.dv) continue;
    const size_t row = (size_t)h * a.dv + r;
    float x[EPL], t[EPL];
    load_f32(x, a.S + row * DK + col0);
#pragma unroll
    for (int e = 0; e < EPL; ++e)
      t[e] = __builtin_amdgcn_fmed3f(fmaf(x[e], inv, F::MQ), F::MQ - F::QMAX, F::MQ + F::QMAX);
    uint32_t X[NW];
    pack_offsets<BITS>(t, X);
    uint8_t* cp = a.codes + row * ROWB + lc * (EPL * BITS / 8);
#pragma unroll
    for (int c = 0; c < NW / 4; ++c)
      *reinterpret_cast<uint4*>(cp + 16 * c) = make_uint4(X[4 * c] ^ F::OFF, X[4 * c + 1] ^ F::OFF,
                                                         X[4 * c + 2] ^ F::OFF, X[4 * c + 3] ^ F::OFF);
  }
  if (tid == 0) a.scales[h] = s;
}

}  // namespace dev

hipError_t launch_head_scale(const StepArgs& a, int bits, int dk, int policy, int rounding,
                             int delta, int diag, hipStream_t s) {
  // heads of at most sixteen row-iterations: one per wave (eight or sixteen
  // waves), the rows held in registers
  const int rpi = 64 / (dk / dev::EPL);
  if (policy == dev::POL_DYNAMIC && a.dv <= 16 * rpi) {
    const bool w8 = a.dv <= 8 * rpi;
    const dim3 grid1(a.n_heads), block1(w8 ? 512 : 1024);
#define LSQ_HS1(B, DK, R, D, G)                                                                 \
    if (bits == B && dk == DK && rounding == R && delta == D && diag == G) {                    \
      if (w8)                                                                                   \
        hipLaunchKernelGGL((dev::head_scale1_kernel<B, DK, R, D, G, 8>), grid1, block1, 0, s, a); \
      else                                                                                      \
        hipLaunchKernelGGL((dev::head_scale1_kernel<B, DK, R, D, G, 16>), grid1, block1, 0, s, a); \
      return hipGetLastError();                                                                 \
    }
#define LSQ_HS1_R(B, DK, R) LSQ_HS1(B, DK, R, 0, 0) LSQ_HS1(B, DK, R, 0, 1) LSQ_HS1(B, DK, R, 1, 0) LSQ_HS1(B, DK, R, 1, 1)
#define LSQ_HS1_DK(B, DK) LSQ_HS1_R(B, DK, dev::RND_RNE) LSQ_HS1_R(B, DK, dev::RND_BDR)
    LSQ_HS1_DK(4, 128) LSQ_HS1_DK(4, 64) LSQ_HS1_DK(8, 128) LSQ_HS1_DK(8, 64)
#undef LSQ_HS1_DK
#undef LSQ_HS1_R
#undef LSQ_HS1
    return hipErrorInvalidValue;
  }
  const dim3 grid(a.n_heads), block(64 * dev::kHeadWaves);
#define LSQ_HS(B, DK, P, R, D, G)                                                               \
  if (bits == B && dk == DK && policy == P && rounding == R && delta == D && diag == G) {      \
    hipLaunchKernelGGL((dev::head_scale_kernel<B, DK, P, R, D, G>), grid, block, 0, s, a);     \
    return hipGetLastError();                                                                   \
  }
#define LSQ_HS_R(B, DK, P, R) LSQ_HS(B, DK, P, R, 0, 0) LSQ_HS(B, DK, P, R, 0, 1) LSQ_HS(B, DK, P, R, 1, 0) LSQ_HS(B, DK, P, R, 1, 1)
#define LSQ_HS_P(B, DK, P) LSQ_HS_R(B, DK, P, dev::RND_RNE) LSQ_HS_R(B, DK, P, dev::RND_BDR)
#define LSQ_HS_DK(B, DK) LSQ_HS_P(B, DK, dev::POL_DYNAMIC)
  LSQ_HS_DK(4, 128) LSQ_HS_DK(4, 64) LSQ_HS_DK(8, 128) LSQ_HS_DK(8, 64)
#undef LSQ_HS_DK
#undef LSQ_HS_P
#undef LSQ_HS_R
#undef LSQ_HS
  return hipErrorInvalidValue;
}

hipError_t launch_calibrate_head(const CalibArgs& a, int bits, int dk, hipStream_t s) {
  const dim3 grid(a.n_heads), block(64 * dev::kHeadWaves);
  if (bits == 4 && dk == 128) hipLaunchKernelGGL((dev::calibrate_head_kernel<4, 128>), grid, block, 0, s, a);
  else if (bits == 4 && dk == 64) hipLaunchKernelGGL((dev::calibrate_head_kernel<4, 64>), grid, block, 0, s, a);
  else if (bits == 8 && dk == 128) hipLaunchKernelGGL((dev::calibrate_head_kernel<8, 128>), grid, block, 0, s, a);
  else if (bits == 8 && dk == 64) hipLaunchKernelGGL((dev::calibrate_head_kernel<8, 64>), grid, block, 0, s, a);
  else return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace lsq
