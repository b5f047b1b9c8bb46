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
// Per-element code (no oriented frame) in the main step kernel's launch
// geometry: one wave per (head, row slice), 32 consecutive elements of a row
// per lane; groups of 32 or more elements, fp32 scales.  k, q and a diagonal
// decay are staged in LDS per wave, row data is addressed from wave-uniform
// head bases, and rows go in pairs with two prefetch buffers.
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
  constexpr int LB = EPL * BITS / 8, WF = 4 * DK;  // code bytes per lane; LDS floats per wave
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(blockIdx.x * 4 + (threadIdx.x >> 6));
  if (wave >= a.total_waves) return;     // whole waves only
  const int h = wave / a.waves_per_head, slice = wave - h * a.waves_per_head;
  const int lr = lane / LPR, lc = lane % LPR, col0 = lc * EPL;
  const uint32_t gi = (uint32_t)(col0 / a.group);   // one group per lane (groups >= 32)
  const uint32_t dv = (uint32_t)a.dv, ng = (uint32_t)a.ng;

  __shared__ float4 lds4[4 * WF / 4];
  float* kv = reinterpret_cast<float*>(lds4) + (threadIdx.x >> 6) * WF;
  float* qv = kv + DK;
  float* av = kv + 2 * DK;
  float* sv = kv + 3 * DK;                       // sign of k_c as +-1, or 0
  if (lr == 0) {
    float x[EPL];
    load_f32(x, a.k + (size_t)h * DK + col0);
    store_lds(kv + col0, x);
#pragma unroll
    for (int e = 0; e < EPL; ++e) x[e] = (float)((x[e] > 0.f) - (x[e] < 0.f));
    store_lds(sv + col0, x);
    load_f32(x, a.q + (size_t)h * DK + col0);
    store_lds(qv + col0, x);
    if constexpr (DIAG) {
      load_f32(x, a.alpha + (size_t)h * DK + col0);
      store_lds(av + col0, x);
    }
  }
  const float alpha_s = DIAG ? 1.f : a.alpha[h];
  const float beta = a.beta[h];
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

  uint8_t* const codes_h = a.codes + (size_t)h * dv * ROWB;
  const float* const scales_h = a.scales + (size_t)h * dv * ng;
  const float* const v_h = a.v + (size_t)h * dv;
  float* const o_h = a.o + (size_t)h * dv;
  struct RowData {
    uint32_t x[NW];
    float s, v;
  };
  auto row_of = [&](int it) -> uint32_t {
    const uint32_t r = (uint32_t)((slice * a.nit + it) * RPI + lr);
    return r < dv ? r : dv - 1;
  };
  auto load_row_data = [&](int it, RowData& d) {
    const uint32_t i = row_of(it);
#pragma unroll
    for (int c = 0; c < NW / 4; ++c) {
      const u32x4 w4 = load_codes16<>(codes_h + (i * ROWB + lc * LB + 16 * c));
      d.x[4 * c] = w4.x; d.x[4 * c + 1] = w4.y; d.x[4 * c + 2] = w4.z; d.x[4 * c + 3] = w4.w;
    }
    d.s = at_bytes(scales_h, (i * ng + gi) * 4u);
    d.v = at_bytes(v_h, i * 4u);
  };

  // One row, from the codes to the packed store.
  auto process = [&](const RowData& cur, int it) {
    const uint32_t r = (uint32_t)((slice * a.nit + it) * RPI + lr);
    const bool live = r < dv;
    const uint32_t i = live ? r : dv - 1;
    int base = col0;                              // laundered: LDS reads stay in the loop
    asm volatile("" : "+v"(base));
    uint32_t xo[NW];
#pragma unroll
    for (int c = 0; c < NW; ++c) xo[c] = cur.x[c] ^ F::OFF;
    // S' = fl(C_old fl(s alpha)) and cold = MQ + C_old (exact), the stored
    // code on the rounding constant's grid
    const float s = cur.s;
    float st[EPL], cold[EPL];
    if constexpr (DIAG) {
      float cu[EPL];                              // offset codes C_old + bias
      unpack_offsets<BITS>(xo, cu);
#pragma unroll
      for (int b = 0; b < EPL / 8; ++b) {
        float ab[8];
        lds_block<DK>(ab, av, base + 8 * b);
#pragma unroll
        for (int e8 = 0; e8 < 8; ++e8) {
          st[8 * b + e8] = (cu[8 * b + e8] - F::BIAS) * (s * ab[e8]);
          cold[8 * b + e8] = cu[8 * b + e8] + (F::MQ - F::BIAS);
        }
      }
    } else {
      const float m[1] = {s * alpha_s}, mb[1] = {-F::BIAS * (s * alpha_s)};
      dequant_mix<BITS, 1>(xo, m, mb, st);
      const float one[1] = {1.f}, mq[1] = {F::MQ - F::BIAS};
      dequant_mix<BITS, 1>(xo, one, mq, cold);
    }
    float u = 0.f;
    if constexpr (DELTA) {
      float pu = 0.f;
#pragma unroll
      for (int b = 0; b < EPL / 8; ++b) {
        float kb[8];
        lds_block<DK>(kb, kv, base + 8 * b);
#pragma unroll
        for (int e8 = 0; e8 < 8; ++e8) pu = fmaf(st[8 * b + e8], kb[e8], pu);
      }
      u = row_sum<LPR>(pu);
    }
    const float w = beta * (cur.v - u);
    float po = 0.f;
#pragma unroll
    for (int b = 0; b < EPL / 8; ++b) {
      float kb[8], qb[8];
      lds_block<DK>(kb, kv, base + 8 * b);
      lds_block<DK>(qb, qv, base + 8 * b);
#pragma unroll
      for (int e8 = 0; e8 < 8; ++e8) {
        st[8 * b + e8] = fmaf(w, kb[e8], st[8 * b + e8]);
        po = fmaf(st[8 * b + e8], qb[e8], po);
      }
    }
    const float o = row_sum<LPR>(po);
    if (live && lc == 0) at_bytes(o_h, i * 4u) = o;

    // c1 = RNE code (offset by MQ, clamped); a reversal is c1 on the far side
    // of C_old from sigma, sigma (C_old - c1) > 0, repaired to c1 + sigma.  With
    // sigma in {-1, 0, 1} as a float and p = sigma (C_old - c1) (exact small
    // integers), the code is fma(med3(p, 0, 1), sigma, c1).  sign(x) as such a
    // float is med3(x 2^200, -1, 1) (two exact scalings: every nonzero float
    // reaches magnitude >= 1); a zero scale has no direction.
    const float inv = inv_scale(s);
    const float on = s > 0.f ? 1.f : 0.f;
    auto sign_of = [](float x) {
      return __builtin_amdgcn_fmed3f((x * 0x1p100f) * 0x1p100f, -1.f, 1.f);
    };
    const float sw = sign_of(w) * on;
    uint32_t X[NW];
#pragma unroll
    for (int b = 0; b < EPL / 8; ++b) {
      float sk[8], t[8];
      if constexpr (VAR == RND_BDR_B) lds_block<DK>(sk, sv, base + 8 * b);
#pragma unroll
      for (int e8 = 0; e8 < 8; ++e8) {
        const int e = 8 * b + e8;
        const float c1 = __builtin_amdgcn_fmed3f(fmaf(st[e], inv, F::MQ), F::MQ - F::QMAX,
                                                 F::MQ + F::QMAX);
        float sigma;
        if constexpr (VAR == RND_BDR_A)
          sigma = sign_of(fmaf(F::MQ - cold[e], s, st[e])) * on;   // sign(S - C_old s)
        else
          sigma = sw * sk[e8];                                      // sign(w) sign(k_c)
        const float p = sigma * (cold[e] - c1);
        t[e8] = fmaf(__builtin_amdgcn_fmed3f(p, 0.f, 1.f), sigma, c1);
      }
      pack_block<BITS>(t, &X[(NW / 4) * b]);
    }
    if (live) {
#pragma unroll
      for (int c = 0; c < NW / 4; ++c)
        store_codes16(codes_h + (i * ROWB + lc * LB + 16 * c),
                      u32x4{X[4 * c] ^ F::OFF, X[4 * c + 1] ^ F::OFF, X[4 * c + 2] ^ F::OFF,
                            X[4 * c + 3] ^ F::OFF});
    }
  };

  // Rows in pairs with two prefetch buffers (no register copies between rows).
  RowData bufA, bufB;
  load_row_data(0, bufA);
  for (int it = 0; it < a.nit; it += 2) {
    if (it + 1 < a.nit) load_row_data(it + 1, bufB);
    process(bufA, it);
    if (it + 1 >= a.nit) break;
    if (it + 2 < a.nit) load_row_data(it + 2, bufA);
    process(bufB, it + 1);
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
