// Decode-step kernels for the quantised recurrent state (gfx950, wave64).
//
// Work decomposition.  Eq. (1) of the LinQuant summary (Theoretical
// Foundation), S_t = S' (I - delta beta k k^T) + beta v k^T with S' = S_{t-1}
// Lambda_t, touches each state row independently:
//     S_t[r,:] = S'[r,:] + w_r k^T,   w_r = beta (v_r - delta S'[r,:] . k),
// so a row needs only its own codes, its scales and the per-head vectors.
// One wavefront owns a slice of rows of one (batch, head).  Each lane owns 16
// contiguous bytes of a packed row: 32 INT4 or 16 INT8 elements, i.e. one
// whole INT4 group of 32 or a quarter of an INT8 group of 64.  LPR lanes
// cover one row, so a wave covers 64/LPR rows per iteration with perfectly
// coalesced 16-byte loads (the wave reads 1 KiB of consecutive codes).  The
// lane keeps k, q (and a diagonal decay) for its columns in registers for all
// rows it visits.  The two row dot products and the group absmax are reduced
// across the LPR lanes of a row with DPP butterflies; no LDS, no atomics, no
// inter-wave communication.  Every step re-reads and re-writes the whole
// packed state from HBM.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "lsq_internal.h"

namespace lsq {
namespace dev {

enum { POL_DYNAMIC = 1, POL_PERSISTENT = 2, POL_YOKED = 3 };
enum { RND_RNE = 0, RND_BDR = 1 };

// 1.5 * 2^23: adding it to |y| < 2^22 with one rounding leaves
// round-half-even(y) in the low mantissa bits (spacing 1 in [2^23, 2^24)).
constexpr float kMagic = 12582912.0f;

// DPP moves (row-local lane permutations, full rate, no LDS).
template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), CTRL, 0xF, 0xF, false));
}
constexpr int kQuadXor1 = 0xB1;       // quad_perm [1,0,3,2]
constexpr int kQuadXor2 = 0x4E;       // quad_perm [2,3,0,1]
constexpr int kRowHalfMirror = 0x141; // lane i <-> 7-i within each 8-lane half-row
constexpr int kRowMirror = 0x140;     // lane i <-> 15-i within each 16-lane row

// Sum over the LPR consecutive lanes of a row.  Butterfly: every lane of the
// row ends with the bitwise same value (fp addition is commutative).
template <int LPR>
__device__ __forceinline__ float row_sum(float x) {
  static_assert(LPR == 1 || LPR == 2 || LPR == 4 || LPR == 8 || LPR == 16, "lanes per row");
  if constexpr (LPR >= 2) x += dpp<kQuadXor1>(x);
  if constexpr (LPR >= 4) x += dpp<kQuadXor2>(x);
  if constexpr (LPR >= 8) x += dpp<kRowHalfMirror>(x);
  if constexpr (LPR >= 16) x += dpp<kRowMirror>(x);
  return x;
}

// Max over an aligned group of gl consecutive lanes (gl a power of two <= 16).
__device__ __forceinline__ float group_max(float x, int gl) {
  if (gl >= 2) x = fmaxf(x, dpp<kQuadXor1>(x));
  if (gl >= 4) x = fmaxf(x, dpp<kQuadXor2>(x));
  if (gl >= 8) x = fmaxf(x, dpp<kRowHalfMirror>(x));
  if (gl >= 16) x = fmaxf(x, dpp<kRowMirror>(x));
  return x;
}

__device__ __forceinline__ float fsign(float x) { return (x > 0.f) ? 1.f : ((x < 0.f) ? -1.f : 0.f); }

template <int N>
__device__ __forceinline__ void load_f32(float (&dst)[N], const float* __restrict__ src) {
  static_assert(N % 4 == 0, "vector loads");
#pragma unroll
  for (int i = 0; i < N / 4; ++i) {
    float4 t = reinterpret_cast<const float4*>(src)[i];
    dst[4 * i + 0] = t.x;
    dst[4 * i + 1] = t.y;
    dst[4 * i + 2] = t.z;
    dst[4 * i + 3] = t.w;
  }
}

template <int N>
__device__ __forceinline__ void store_f32(float* __restrict__ dst, const float (&src)[N]) {
#pragma unroll
  for (int i = 0; i < N / 4; ++i)
    reinterpret_cast<float4*>(dst)[i] = make_float4(src[4 * i], src[4 * i + 1], src[4 * i + 2],
                                                    src[4 * i + 3]);
}

// Signed code of element e (0 <= e < 128/BITS) of a 16-byte lane chunk.
template <int BITS>
__device__ __forceinline__ int code_at(const uint32_t (&w)[4], int e) {
  if constexpr (BITS == 4) {
    const uint32_t word = w[e >> 3];
    return static_cast<int>(word << (28 - 4 * (e & 7))) >> 28;
  } else {
    const uint32_t word = w[e >> 2];
    return static_cast<int>(word << (24 - 8 * (e & 3))) >> 24;
  }
}

template <int BITS, int DK, int POLICY, int ROUND, int DELTA, int DIAG>
__global__ __launch_bounds__(256) void step_kernel(StepArgs a) {
  constexpr int EPL = 128 / BITS;        // elements per lane: 16 bytes of codes
  constexpr int LPR = DK / EPL;          // lanes per row
  constexpr int RPI = 64 / LPR;          // rows per wave-iteration
  constexpr int ROWB = DK * BITS / 8;    // packed bytes per row
  constexpr float QMAX = float((1 << (BITS - 1)) - 1);
  static_assert(LPR >= 1 && LPR <= 16, "row must fit a 16-lane DPP row");

  const int lane = threadIdx.x & 63;
  const int wave = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (wave >= a.total_waves) return;     // whole waves only
  const int h = wave / a.waves_per_head;
  const int slice = wave - h * a.waves_per_head;
  const int lr = lane / LPR;
  const int lc = lane % LPR;
  const int col0 = lc * EPL;
  const int gl = a.group / EPL;          // lanes per group (>= 1)
  const int gi = col0 / a.group;         // this lane's group

  // per-head vectors for this lane's columns
  float kk[EPL], qq[EPL];
  load_f32(kk, a.k + (size_t)h * DK + col0);
  load_f32(qq, a.q + (size_t)h * DK + col0);
  float aa[DIAG ? EPL : 4];
  if constexpr (DIAG) load_f32(aa, a.alpha + (size_t)h * DK + col0);
  const float alpha_s = DIAG ? 1.f : a.alpha[h];
  const float beta = a.beta[h];

  for (int it = 0; it < a.nit; ++it) {
    const int r = (slice * a.nit + it) * RPI + lr;
    const bool live = r < a.dv;          // uniform over the lanes of a row
    const size_t row = (size_t)h * a.dv + (live ? r : a.dv - 1);

    const uint4 cw = *reinterpret_cast<const uint4*>(a.codes + row * ROWB + lc * 16);
    const uint32_t words[4] = {cw.x, cw.y, cw.z, cw.w};
    const float s = a.scales[row * a.ng + gi];
    const float vr = a.v[row];

    // dequantise with the decay folded into the group scale: S' = C * fl(s*alpha)
    float sp[EPL];
    const float ms = s * alpha_s;
#pragma unroll
    for (int e = 0; e < EPL; ++e) {
      const float m = DIAG ? s * aa[e] : ms;
      sp[e] = static_cast<float>(code_at<BITS>(words, e)) * m;
    }

    // delta correction u = S' . k and the write coefficient w = beta (v - u)
    float u = 0.f;
    if constexpr (DELTA) {
      float p = 0.f;
#pragma unroll
      for (int e = 0; e < EPL; ++e) p = fmaf(sp[e], kk[e], p);
      u = row_sum<LPR>(p);
    }
    const float w = beta * (vr - u);

    // rank-one write and readout o_r = S_t . q (before requantisation)
    float st[EPL];
    float po = 0.f;
#pragma unroll
    for (int e = 0; e < EPL; ++e) {
      st[e] = fmaf(w, kk[e], sp[e]);
      po = fmaf(st[e], qq[e], po);
    }
    const float o = row_sum<LPR>(po);
    if (live && lc == 0) a.o[row] = o;

    // yoked arm: advance the fp32 reference row with the same update
    float amax_src = 0.f;
    if constexpr (POLICY == POL_YOKED) {
      float R[EPL];
      float* rp = a.ref + row * DK + col0;
      load_f32(R, rp);
#pragma unroll
      for (int e = 0; e < EPL; ++e) R[e] = R[e] * (DIAG ? aa[e] : alpha_s);
      float ur = 0.f;
      if constexpr (DELTA) {
        float p = 0.f;
#pragma unroll
        for (int e = 0; e < EPL; ++e) p = fmaf(R[e], kk[e], p);
        ur = row_sum<LPR>(p);
      }
      const float wr = beta * (vr - ur);
      float pr = 0.f;
#pragma unroll
      for (int e = 0; e < EPL; ++e) {
        R[e] = fmaf(wr, kk[e], R[e]);
        pr = fmaf(R[e], qq[e], pr);
        amax_src = fmaxf(amax_src, fabsf(R[e]));
      }
      const float oref = row_sum<LPR>(pr);
      if (live) {
        store_f32(rp, R);
        if (lc == 0 && a.o_ref) a.o_ref[row] = oref;
      }
    } else if constexpr (POLICY == POL_DYNAMIC) {
#pragma unroll
      for (int e = 0; e < EPL; ++e) amax_src = fmaxf(amax_src, fabsf(st[e]));
    }

    // scale policy
    float snew = s;
    if constexpr (POLICY != POL_PERSISTENT) {
      const float amax = group_max(amax_src, gl);
      snew = amax / QMAX;                       // IEEE division
    }
    const float inv = (snew == 0.f) ? 0.f : 1.0f / snew;

    // requantise: round half to even of the exact product, clamp, then BDR
    const float wsgn = fsign(w);
    uint32_t out[4] = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int e = 0; e < EPL; ++e) {
      float t = fmaf(st[e], inv, kMagic);
      t = __builtin_amdgcn_fmed3f(t, kMagic - QMAX, kMagic + QMAX);
      float c = t - kMagic;
      if constexpr (ROUND == RND_BDR) {
        const float sg = wsgn * fsign(kk[e]);
        const float d = fmaf(sp[e], -inv, c);   // exact sign of c - S'*inv
        if ((sg > 0.f && d < 0.f) || (sg < 0.f && d > 0.f))
          c = fminf(fmaxf(c + sg, -QMAX), QMAX);
      }
      const uint32_t ci = static_cast<uint32_t>(static_cast<int>(c));
      if constexpr (BITS == 4)
        out[e >> 3] |= (ci & 0xFu) << (4 * (e & 7));
      else
        out[e >> 2] |= (ci & 0xFFu) << (8 * (e & 3));
    }
    if (live) {
      *reinterpret_cast<uint4*>(a.codes + row * ROWB + lc * 16) =
          make_uint4(out[0], out[1], out[2], out[3]);
      if constexpr (POLICY != POL_PERSISTENT) {
        if ((lc % gl) == 0) a.scales[row * a.ng + gi] = snew;
      }
    }
  }
}

// Dispatch one (BITS, DK) family over the method flags.
template <int BITS, int DK>
hipError_t launch_family(const StepArgs& a, int policy, int rounding, int delta, int diag,
                         hipStream_t s) {
  const dim3 grid((a.total_waves + 3) / 4), block(256);
#define LSQ_CASE(P, R, D, G)                                                               \
  if (policy == P && rounding == R && delta == D && diag == G) {                           \
    hipLaunchKernelGGL((step_kernel<BITS, DK, P, R, D, G>), grid, block, 0, s, a);         \
    return hipGetLastError();                                                              \
  }
#define LSQ_CASES_PR(P, R) \
  LSQ_CASE(P, R, 0, 0) LSQ_CASE(P, R, 0, 1) LSQ_CASE(P, R, 1, 0) LSQ_CASE(P, R, 1, 1)
#define LSQ_CASES_P(P) LSQ_CASES_PR(P, RND_RNE) LSQ_CASES_PR(P, RND_BDR)
  LSQ_CASES_P(POL_DYNAMIC)
  LSQ_CASES_P(POL_PERSISTENT)
  LSQ_CASES_P(POL_YOKED)
#undef LSQ_CASES_P
#undef LSQ_CASES_PR
#undef LSQ_CASE
  return hipErrorInvalidValue;
}

}  // namespace dev
}  // namespace lsq
