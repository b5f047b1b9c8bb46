// Decode step with the two readings of directional rounding that the library
// does not take, kept behind rounding flags for sensitivity runs.
//
// "Preserving Updates in Low-Bit Recurrent State Quantization" (abstract)
// says an element can move opposite to its update and that directional
// rounding sends such elements toward their updates, without defining the
// update or the move.  The default reading (LSQ_ROUND_BDR) measures the move
// from the decayed pre-write value against the rank-one write.  The two
// readings here, under a frozen (persistent) scale, compare the new code with
// the stored code C_old, which lies on this step's grid:
//   A   update = the total change from the stored value:
//       sigma = sign(S - C_old s), exact as the sign of one fma;
//   B'  update = the rank-one write, sigma = sign(w) sign(k_c);
// a reversal is a round-to-nearest-even code c1 on the far side of C_old
// from sigma, replaced by c1 + sigma (which stays between c1 and C_old).
//
// Plain per-element code (no oriented frame): one wave per (head, row slice),
// 32 consecutive elements of a row per lane, the launch geometry of the main
// step kernel; groups of 32 or more elements, fp32 scales.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "lsq_step_impl.h"

namespace lsq {
namespace dev {

constexpr int RND_BDR_A = 3, RND_BDR_B = 4;

template <int BITS, int DK, int VAR, int DELTA, int DIAG>
__global__ __launch_bounds__(256) void bdr_alt_kernel(StepArgs a) {
  using F = Fmt<BITS>;
  constexpr int NW = F::NW, LPR = DK / EPL, RPI = 64 / LPR, ROWB = DK * BITS / 8;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(blockIdx.x * 4 + (threadIdx.x >> 6));
  if (wave >= a.total_waves) return;     // whole waves only
  const int h = wave / a.waves_per_head, slice = wave - h * a.waves_per_head;
  const int lr = lane / LPR, lc = lane % LPR, col0 = lc * EPL;
  const int gi = col0 / a.group;         // one group per lane (groups >= 32)

  float kk[EPL], qq[EPL], al[DIAG ? EPL : 4];
  load_f32(kk, a.k + (size_t)h * DK + col0);
  load_f32(qq, a.q + (size_t)h * DK + col0);
  if constexpr (DIAG) load_f32(al, a.alpha + (size_t)h * DK + col0);
  else al[0] = a.alpha[h];
  const float beta = a.beta[h];

  for (int it = 0; it < a.nit; ++it) {
    const int r = (slice * a.nit + it) * RPI + lr;
    const bool live = r < a.dv;
    const size_t row = (size_t)h * a.dv + (live ? r : a.dv - 1);
    uint8_t* cp = a.codes + row * ROWB + lc * (EPL * BITS / 8);
    uint32_t xo[NW];
#pragma unroll
    for (int c = 0; c < NW / 4; ++c) {
      const u32x4 w4 = load_codes16(cp + 16 * c);
      xo[4 * c + 0] = w4.x ^ F::OFF;
      xo[4 * c + 1] = w4.y ^ F::OFF;
      xo[4 * c + 2] = w4.z ^ F::OFF;
      xo[4 * c + 3] = w4.w ^ F::OFF;
    }
    float cu[EPL];                       // offset codes C_old + bias
    unpack_offsets<BITS>(xo, cu);
    const float s = a.scales[row * a.ng + gi];
    float sp[EPL];
    float pu = 0.f;
#pragma unroll
    for (int e = 0; e < EPL; ++e) {
      const float m = s * (DIAG ? al[e] : al[0]);
      sp[e] = (cu[e] - F::BIAS) * m;     // S' = fl(C_old fl(s alpha))
      if constexpr (DELTA) pu = fmaf(sp[e], kk[e], pu);
    }
    const float u = DELTA ? row_sum<LPR>(pu) : 0.f;
    const float w = beta * (a.v[row] - u);
    float st[EPL];
    float po = 0.f;
#pragma unroll
    for (int e = 0; e < EPL; ++e) {
      st[e] = fmaf(w, kk[e], sp[e]);
      po = fmaf(st[e], qq[e], po);
    }
    const float o = row_sum<LPR>(po);
    if (live && lc == 0) a.o[row] = o;

    const float inv = inv_scale(s);
    const bool on = s > 0.f;
    const int sw = (w > 0.f) - (w < 0.f);
    float t[EPL];
#pragma unroll
    for (int e = 0; e < EPL; ++e) {
      // MQ + RNE(S inv), clamped: the offset code in the low mantissa bits
      const float c1 = __builtin_amdgcn_fmed3f(fmaf(st[e], inv, F::MQ), F::MQ - F::QMAX,
                                               F::MQ + F::QMAX);
      const float cold = cu[e] + (F::MQ - F::BIAS);   // MQ + C_old, exact
      int sigma;
      if constexpr (VAR == RND_BDR_A) {
        const float d = fmaf(F::BIAS - cu[e], s, st[e]);   // S - C_old s, one rounding
        sigma = (d > 0.f) - (d < 0.f);
      } else {
        sigma = sw * ((kk[e] > 0.f) - (kk[e] < 0.f));
      }
      const bool rev = on && ((sigma > 0 && c1 < cold) || (sigma < 0 && c1 > cold));
      t[e] = rev ? c1 + (float)sigma : c1;
    }
    uint32_t X[NW];
    pack_offsets<BITS>(t, X);
    if (live) {
#pragma unroll
      for (int c = 0; c < NW / 4; ++c)
        store_codes16(cp + 16 * c, u32x4{X[4 * c] ^ F::OFF, X[4 * c + 1] ^ F::OFF,
                                         X[4 * c + 2] ^ F::OFF, X[4 * c + 3] ^ F::OFF});
    }
  }
}

}  // namespace dev

hipError_t launch_bdr_alt(const StepArgs& a, int bits, int dk, int rounding, int delta, int diag,
                          hipStream_t s) {
  const dim3 grid((a.total_waves + 3) / 4), block(256);
#define LSQ_BA(B, DK, V, D, G)                                                                \
  if (bits == B && dk == DK && rounding == V && delta == D && diag == G) {                   \
    hipLaunchKernelGGL((dev::bdr_alt_kernel<B, DK, V, D, G>), grid, block, 0, s, a);         \
    return hipGetLastError();                                                                 \
  }
#define LSQ_BA_V(B, DK, V) LSQ_BA(B, DK, V, 0, 0) LSQ_BA(B, DK, V, 0, 1) LSQ_BA(B, DK, V, 1, 0) LSQ_BA(B, DK, V, 1, 1)
#define LSQ_BA_DK(B, DK) LSQ_BA_V(B, DK, dev::RND_BDR_A) LSQ_BA_V(B, DK, dev::RND_BDR_B)
  LSQ_BA_DK(4, 128) LSQ_BA_DK(4, 64) LSQ_BA_DK(8, 128) LSQ_BA_DK(8, 64)
#undef LSQ_BA_DK
#undef LSQ_BA_V
#undef LSQ_BA
  return hipErrorInvalidValue;
}

}  // namespace lsq
