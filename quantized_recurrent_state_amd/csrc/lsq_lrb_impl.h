// Decode step with Low-Rank Bypass (a rank-r fp32 buffer of the last writes,
// merged into the quantised state every r steps).
//
// Reading of the bypass sentence of "Preserving Updates in Low-Bit Recurrent
// State Quantization" (abstract) that this kernel implements (the same as the
// oracle's): slot j of a head holds a_j [Dv] and b_j [Dk], B = sum_j a_j b_j^T;
// the buffer decays with the state (scalar decay scales a_j, diagonal decay
// scales b_j, one fp32 product per step); a step's write w k^T fills the next
// slot (a = w, b = k) instead of entering the quantised state; the delta
// projection and the readout see S' + B; on every r-th step the buffer is
// merged, X = S' + sum_j a_j b_j built by fmas in slot order, requantised under
// the scale policy and rounding (directional rounding takes the sign of the
// buffer's own value U = sum_j a_j b_j, fmas from 0), and emptied.  Between
// merges the state is requantised from S' alone.
//
// Work decomposition as in the plain step: one wave per (head, row slice), 32
// consecutive elements of a row per lane.  The head's vectors and its decayed
// b_j sit in LDS; the slot projections b_j . k, b_j . q and k . q are reduced
// once per wave and, being the same on every lane, kept in scalar registers.
// Row data (codes, scale, v and the row's a_j) is addressed from wave-uniform
// head bases; rows go in pairs with two prefetch buffers, so the next row's
// loads are in flight while a row is computed.  On a merge step under a frozen scale
// each block of eight elements is merged, rounded and packed before the next
// is built, so X and U never occupy more than a block's registers.  Buffer
// memory per head: a [r][Dv]; b [2][r][Dk], the second copy used by diagonal
// decay, which rewrites the decayed b_j each step into the copy the next step
// reads (other waves of the head still read this step's copy).
//
// RMAX (4 or 8) bounds the rank an instance serves: the per-slot registers
// (a_j of the current and the next row, the decayed a'_j, the projections)
// scale with it, and ranks up to 4 take the smaller instance.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "lsq_step_impl.h"

namespace lsq {
namespace dev {

// A float that every lane of the wave holds with the same bits, as a scalar.
__device__ __forceinline__ float wave_uniform(float x) {
  return __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(x)));
}

// fn(std::integral_constant<int, c>) for the c in [0, N) equal to count.
template <int N, typename Fn>
__device__ __forceinline__ void dispatch_count(int count, Fn&& fn) {
  if constexpr (N > 0) {
    if (count == N - 1)
      fn(std::integral_constant<int, N - 1>{});
    else
      dispatch_count<N - 1>(count, fn);
  }
}

// MERGE: this step fills the last slot and merges (a separate instance, so
// that the other steps carry none of the merge's registers).
template <int BITS, int DK, int POLICY, int ROUND, int DELTA, int DIAG, bool MERGE, int RMAX>
__global__ __launch_bounds__(256) void lrb_step_kernel(StepArgs a) {
  using F = Fmt<BITS>;
  constexpr int NW = F::NW, WPB = NW / 4;          // code words per lane, per 8 elements
  constexpr int LPR = DK / EPL, RPI = 64 / LPR, ROWB = DK * BITS / 8, LB = EPL * BITS / 8;
  constexpr int WF = (3 + RMAX) * DK;              // LDS floats per wave: k, q, alpha, b'_0..
  constexpr bool BDR_MERGE = MERGE && ROUND == RND_BDR;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(blockIdx.x * 4 + (threadIdx.x >> 6));
  if (wave >= a.total_waves) return;
  const int h = wave / a.waves_per_head;
  const int slice = wave - h * a.waves_per_head;
  const int lr = lane / LPR, lc = lane % LPR, col0 = lc * EPL;
  const int gl = a.group / EPL, gi = col0 / a.group;
  const int R = a.lrb_rank, nu = a.lrb_used;       // slots filled before this step
  const uint32_t dv = (uint32_t)a.dv, ng = (uint32_t)a.ng;

  __shared__ float4 lds4[4 * WF / 4];
  float* vec = reinterpret_cast<float*>(lds4) + (threadIdx.x >> 6) * WF;
  float* kv = vec;
  float* qv = vec + DK;
  float* av = vec + 2 * DK;
  float* bv = vec + 3 * DK;                        // b'_j at bv + j*DK

  const size_t hk = (size_t)h * DK;
  float kk[EPL], qq[EPL], aa[DIAG ? EPL : 1];
  load_f32(kk, a.k + hk + col0);
  load_f32(qq, a.q + hk + col0);
  if constexpr (DIAG) load_f32(aa, a.alpha + hk + col0);
  const float alpha_s = DIAG ? 1.f : a.alpha[h];
  const float beta = a.beta[h];
  const bool writer = lr == 0;
  if (writer) {
    store_lds(kv + col0, kk);
    store_lds(qv + col0, qq);
    if constexpr (DIAG) store_lds(av + col0, aa);
  }
  // decayed slots b'_j (j < nu), their projections, and k . q
  float* bh_in = a.lrb_b + ((size_t)h * 2 + a.lrb_cin) * R * DK;
  float* bh_out = a.lrb_b + ((size_t)h * 2 + a.lrb_cout) * R * DK;
  float bk[RMAX], bq[RMAX];
#pragma unroll
  for (int j = 0; j < RMAX; ++j) {
    bk[j] = bq[j] = 0.f;
    if (j >= nu) continue;
    float b[EPL];
    load_f32(b, bh_in + (size_t)j * DK + col0);
    if constexpr (DIAG) {
#pragma unroll
      for (int e = 0; e < EPL; ++e) b[e] = b[e] * aa[e];
    }
    float pk = 0.f, pq = 0.f;
#pragma unroll
    for (int e = 0; e < EPL; ++e) {
      pk = fmaf(b[e], kk[e], pk);
      pq = fmaf(b[e], qq[e], pq);
    }
    // every row of lanes reduces the same values in the same order
    bk[j] = wave_uniform(row_sum<LPR>(pk));
    bq[j] = wave_uniform(row_sum<LPR>(pq));
    if (writer) {
      store_lds(bv + j * DK + col0, b);
      if (DIAG && !MERGE && slice == 0) store_f32(bh_out + (size_t)j * DK + col0, b);
    }
  }
  float pkq = 0.f;
#pragma unroll
  for (int e = 0; e < EPL; ++e) pkq = fmaf(kk[e], qq[e], pkq);
  const float kq = wave_uniform(row_sum<LPR>(pkq));
  // the new slot's b is k (written where the next step reads it)
  if (!MERGE && slice == 0 && writer) store_f32(bh_out + (size_t)nu * DK + col0, kk);
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

  // wave-uniform bases of the head's rows; a lane adds a 32-bit byte offset
  uint8_t* const codes_h = a.codes + (size_t)h * dv * ROWB;
  float* const scales_h = a.scales + (size_t)h * dv * ng;
  const float* const v_h = a.v + (size_t)h * dv;
  float* const o_h = a.o + (size_t)h * dv;
  float* const ah = a.lrb_a + (size_t)h * R * dv;  // a_j[i] at ah[j*dv + i]
  struct RowData {
    uint32_t x[NW];
    float s, v;
    float aj[RMAX];
  };
  auto row_of = [&](int it) -> uint32_t {
    const uint32_t r = (uint32_t)((slice * a.nit + it) * RPI + lr);
    return r < dv ? r : dv - 1;
  };
  auto load_row_data = [&](int it, RowData& d) {
    const uint32_t i = row_of(it);
    const uint8_t* p = codes_h + (i * ROWB + lc * LB);
#pragma unroll
    for (int c = 0; c < NW / 4; ++c) {
      const u32x4 w4 = load_codes16<>(p + 16 * c);
      d.x[4 * c] = w4.x; d.x[4 * c + 1] = w4.y; d.x[4 * c + 2] = w4.z; d.x[4 * c + 3] = w4.w;
    }
    d.s = at_bytes(scales_h, (i * ng + gi) * 4u);
    d.v = at_bytes(v_h, i * 4u);
#pragma unroll
    for (int j = 0; j < RMAX; ++j) d.aj[j] = (j < nu) ? at_bytes(ah, ((uint32_t)j * dv + i) * 4u) : 0.f;
  };
  // One row, from dequantisation to the packed store.
  auto process = [&](const RowData& cur, int it) {
    const uint32_t r = (uint32_t)((slice * a.nit + it) * RPI + lr);
    const bool live = r < dv;
    const uint32_t i = live ? r : dv - 1;
    int base = col0;                              // laundered: LDS reads stay in the loop
    asm volatile("" : "+v"(base));
    // codes -> S' (decay folded into the scale)
    uint32_t x[NW];
#pragma unroll
    for (int c = 0; c < NW; ++c) x[c] = cur.x[c] ^ F::OFF;
    const float s = cur.s;
    float sp[EPL];
    if constexpr (DIAG) {
      unpack_offsets<BITS>(x, sp);
#pragma unroll
      for (int b = 0; b < EPL / 8; ++b) {
        float ab[8];
        lds_block<DK>(ab, av, base + 8 * b);
#pragma unroll
        for (int e8 = 0; e8 < 8; ++e8) sp[8 * b + e8] = (sp[8 * b + e8] - F::BIAS) * (s * ab[e8]);
      }
    } else {
      const float m[1] = {s * alpha_s}, mb[1] = {-F::BIAS * (s * alpha_s)};
      dequant_mix<BITS, 1>(x, m, mb, sp);
    }
    // decayed a'_j of this row
    float ap[RMAX];
#pragma unroll
    for (int j = 0; j < RMAX; ++j) ap[j] = DIAG ? cur.aj[j] : cur.aj[j] * alpha_s;
    // delta projection on S' + B', the write coefficient, the readout
    float u = 0.f;
    if constexpr (DELTA) {
      float p = 0.f;
#pragma unroll
      for (int b = 0; b < EPL / 8; ++b) {
        float kb[8];
        lds_block<DK>(kb, kv, base + 8 * b);
#pragma unroll
        for (int e8 = 0; e8 < 8; ++e8) p = fmaf(sp[8 * b + e8], kb[e8], p);
      }
      u = row_sum<LPR>(p);
#pragma unroll
      for (int j = 0; j < RMAX; ++j)
        if (j < nu) u = fmaf(ap[j], bk[j], u);
    }
    const float w = beta * (cur.v - u);
    float po = 0.f;
#pragma unroll
    for (int b = 0; b < EPL / 8; ++b) {
      float qb[8];
      lds_block<DK>(qb, qv, base + 8 * b);
#pragma unroll
      for (int e8 = 0; e8 < 8; ++e8) po = fmaf(sp[8 * b + e8], qb[e8], po);
    }
    float o = row_sum<LPR>(po);
#pragma unroll
    for (int j = 0; j < RMAX; ++j)
      if (j < nu) o = fmaf(ap[j], bq[j], o);
    o = fmaf(w, kq, o);
    if (live && lc == 0) at_bytes(o_h, i * 4u) = o;

    // Requantisation of the row into X4.  On a merge step the number of slots
    // to merge, NU, is a compile-time constant (one copy of this code per
    // value, chosen by the wave-uniform slot count), so the merge is
    // straight-line code.
    uint32_t X4[NW];
    float snew = s;
    int mbase = col0;                             // a second laundered offset: k is
    asm volatile("" : "+v"(mbase));               // re-read, not held since the projection
    auto requant = [&](auto nuc) {
      constexpr int NU = decltype(nuc)::value;
      // Block b of the merged value X = S' + sum_j a'_j b'_j + w k (fmas in
      // slot order) and of the buffer's own value U (the same fmas from 0),
      // which gives directional rounding its direction.
      auto merged = [&](int mb, int b, float (&X8)[8], float (&U8)[8]) {
#pragma unroll
        for (int e8 = 0; e8 < 8; ++e8) {
          X8[e8] = sp[8 * b + e8];
          U8[e8] = 0.f;
        }
#pragma unroll
        for (int jj = 0; jj < NU; ++jj) {
          float bb[8];
          lds_block<DK>(bb, bv, jj * DK + mb + 8 * b);
#pragma unroll
          for (int e8 = 0; e8 < 8; ++e8) {
            X8[e8] = fmaf(ap[jj], bb[e8], X8[e8]);
            if constexpr (BDR_MERGE) U8[e8] = fmaf(ap[jj], bb[e8], U8[e8]);
          }
        }
        float kb[8];
        lds_block<DK>(kb, kv, mb + 8 * b);
#pragma unroll
        for (int e8 = 0; e8 < 8; ++e8) {
          X8[e8] = fmaf(w, kb[e8], X8[e8]);
          if constexpr (BDR_MERGE) U8[e8] = fmaf(w, kb[e8], U8[e8]);
        }
      };

      // The dynamic policy needs the group maximum before any element rounds:
      // on a merge step a first pass builds the merged blocks for their
      // maximum only, and the rounding pass builds them again (the same fmas,
      // so the same values), which keeps X and U to a block's registers.
      if constexpr (POLICY == POL_DYNAMIC) {
        float amax = 0.f;
        if constexpr (MERGE) {
          int mb1 = col0;                         // its own laundered offset: the two
          asm volatile("" : "+v"(mb1));           // passes share no loaded values
#pragma unroll
          for (int b = 0; b < EPL / 8; ++b) {
            float X8[8], U8[8];
            merged(mb1, b, X8, U8);
#pragma unroll
            for (int e8 = 0; e8 < 8; ++e8) amax = fmaxf(amax, fabsf(X8[e8]));
          }
        } else {
#pragma unroll
          for (int e = 0; e < EPL; ++e) amax = fmaxf(amax, fabsf(sp[e]));
        }
        snew = group_max(amax, gl) / F::QMAX;
      }
      const float inv = inv_scale(snew);
#pragma unroll
      for (int b = 0; b < EPL / 8; ++b) {
        float X8[8], U8[8];
        if constexpr (MERGE) {
          merged(mbase, b, X8, U8);
        } else {
#pragma unroll
          for (int e8 = 0; e8 < 8; ++e8) X8[e8] = sp[8 * b + e8];
        }
        float t[8];
        if constexpr (ROUND == RND_DITHER) {
          // floor(z + u) with the Weyl offsets of elements 8b .. 8b+7
          const uint32_t dbase = a.dither_base + i * a.dither_row + (uint32_t)(col0 + 8 * b) * kWeyl;
          float e8[8];
#pragma unroll
          for (int k8 = 0; k8 < 8; ++k8)
            e8[k8] = __uint_as_float(__builtin_amdgcn_alignbit(0x7Fu, dbase + (uint32_t)k8 * kWeyl, 9));
          fma_add_rd8(t, X8, inv, e8, F::MQ - 1.f);
#pragma unroll
          for (int e8 = 0; e8 < 8; ++e8)
            t[e8] = __builtin_amdgcn_fmed3f(t[e8], F::MQ - F::QMAX, F::MQ + F::QMAX);
        } else {
#pragma unroll
          for (int e8 = 0; e8 < 8; ++e8)
            t[e8] = __builtin_amdgcn_fmed3f(fmaf(X8[e8], inv, F::MQ), F::MQ - F::QMAX, F::MQ + F::QMAX);
          if constexpr (BDR_MERGE) {
            // reversal: the rounded code c1 lies on the far side of y' = S' inv
            // from the buffer's update; move it one step toward the update
#pragma unroll
            for (int e8 = 0; e8 < 8; ++e8) {
              const float c1 = t[e8] - F::MQ;                     // exact
              const float d = fmaf(sp[8 * b + e8], inv, -c1);     // sign of y' - c1, exact
              // d times the sign of U (a sign-bit flip), and copysign(1, U)
              const uint32_t su = fbits(U8[e8]) & 0x80000000u;
              const float ds = __uint_as_float(fbits(d) ^ su);
              const float sg = __uint_as_float(0x3F800000u | su);
              const float step = (ds > 0.f && U8[e8] != 0.f) ? sg : 0.f;   // branch-free
              t[e8] = __builtin_amdgcn_fmed3f(t[e8] + step, F::MQ - F::QMAX, F::MQ + F::QMAX);
            }
          }
        }
        pack_block<BITS>(t, &X4[WPB * b]);
      }
    };
    if constexpr (MERGE)
      dispatch_count<RMAX>(nu, requant);
    else
      requant(std::integral_constant<int, 0>{});
    if (live) {
      uint8_t* p = codes_h + (i * ROWB + lc * LB);
#pragma unroll
      for (int c = 0; c < NW / 4; ++c)
        store_codes16(p + 16 * c, u32x4{X4[4 * c] ^ F::OFF, X4[4 * c + 1] ^ F::OFF,
                                        X4[4 * c + 2] ^ F::OFF, X4[4 * c + 3] ^ F::OFF});
      if constexpr (POLICY == POL_DYNAMIC) {
        if ((lc % gl) == 0) at_bytes(scales_h, (i * ng + gi) * 4u) = snew;
      }
      // the buffer: decayed a'_j (scalar decay) and the new slot a_nu = w
      if (!MERGE && lc == 0) {
        if constexpr (!DIAG) {
#pragma unroll
          for (int j = 0; j < RMAX; ++j)
            if (j < nu) at_bytes(ah, ((uint32_t)j * dv + i) * 4u) = ap[j];
        }
        at_bytes(ah, ((uint32_t)nu * dv + i) * 4u) = w;
      }
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

// Dispatch the bypass instances of one rank bound over the method flags.
template <int RMAX>
hipError_t launch_lrb_rmax(const StepArgs& a, int bits, int dk, int policy, int rounding,
                           int delta, int diag, hipStream_t s) {
  const dim3 grid((a.total_waves + 3) / 4), block(256);
#define LSQ_LRB(B, DK, P, RD, D, G)                                                          \
  if (bits == B && dk == DK && policy == P && rounding == RD && delta == D && diag == G) {   \
    if (a.lrb_merge)                                                                        \
      hipLaunchKernelGGL((dev::lrb_step_kernel<B, DK, P, RD, D, G, true, RMAX>), grid, block, 0, s, a); \
    else                                                                                    \
      hipLaunchKernelGGL((dev::lrb_step_kernel<B, DK, P, RD, D, G, false, RMAX>), grid, block, 0, s, a); \
    return hipGetLastError();                                                               \
  }
#define LSQ_LRB_DG(B, DK, P, RD) \
  LSQ_LRB(B, DK, P, RD, 0, 0) LSQ_LRB(B, DK, P, RD, 0, 1) LSQ_LRB(B, DK, P, RD, 1, 0) LSQ_LRB(B, DK, P, RD, 1, 1)
#define LSQ_LRB_R(B, DK, P) \
  LSQ_LRB_DG(B, DK, P, dev::RND_RNE) LSQ_LRB_DG(B, DK, P, dev::RND_BDR) LSQ_LRB_DG(B, DK, P, dev::RND_DITHER)
#define LSQ_LRB_P(B, DK) LSQ_LRB_R(B, DK, dev::POL_DYNAMIC) LSQ_LRB_R(B, DK, dev::POL_PERSISTENT)
  LSQ_LRB_P(4, 128) LSQ_LRB_P(4, 64) LSQ_LRB_P(8, 128) LSQ_LRB_P(8, 64)
#undef LSQ_LRB_P
#undef LSQ_LRB_R
#undef LSQ_LRB_DG
#undef LSQ_LRB
  return hipErrorInvalidValue;
}

}  // namespace lsq
