// Decode-step kernels for the quantised recurrent state (gfx950, wave64).
//
// Work decomposition.  Eq. (1) of the LinQuant summary (Theoretical
// Foundation), S_t = S' (I - delta beta k k^T) + beta v k^T with S' = S_{t-1}
// Lambda_t, touches each state row independently:
//     S_t[r,:] = S'[r,:] + w_r k^T,   w_r = beta (v_r - delta S'[r,:] . k),
// so a row needs only its own codes, its scales and the per-head vectors.
// One wavefront owns a slice of rows of one (batch, head).  Each lane owns 32
// consecutive elements of a row (16 bytes of INT4 or 32 bytes of INT8 codes);
// Dk/32 lanes cover a row, so a wave covers 64/(Dk/32) rows per iteration and
// its loads of codes are consecutive in memory.  The lane keeps k and q (and a
// diagonal decay) for its 32 columns in registers for every row it visits.
// The two row dot products and the group absmax are reduced across the lanes
// of a row with DPP butterflies; no LDS, no atomics, no inter-wave traffic.
// Every step re-reads and re-writes the whole packed state from HBM; the next
// row's codes, scale and v are loaded while the current row is computed.
//
// Instruction budget.  The step is bound by vector-ALU issue, not by the
// matrix cores (it is a batch of matrix-vector updates), so every element
// costs a handful of VALU operations:
//   unpack   offset-binary codes -> v_cvt_f32_ubyteN (nibbles split with two
//            masks; the two's-complement <-> offset-binary flip folds into the
//            same bit operation)
//   S'       one fma per element: fl(C * m) = fma(u, m, -bias*m) exactly, with
//            u = C + bias the offset code and m = fl(s * alpha)
//   u, S, o  three fmas (delta dot, rank-one write, readout)
//   round    fma(S, inv, 1.5*2^23 + bias): the exact product rounded half to
//            even lands in the low mantissa bits, already offset; med3 clamps
//   pack     v_lshl_or / v_perm gather the low bytes
// Bounded directional rounding runs in a sign-oriented frame: the codes of
// columns with k_c < 0 are negated at unpack (a carry-free xor-add on the
// packed offset codes), the sign of w is folded into the sign of inv, so that
// every element's update points upward.  Then the rule "move a reversed code
// one grid step toward its update" equals clamp(max(RNE(z), ceil(z'))) with
// z = S*inv and z' = S'*inv in that frame, i.e. one extra fma rounded toward
// +infinity (MODE register switched around a block of fmas) and one max per
// element.  The packed result is turned back by the same xor-add.
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
constexpr int EPL = 32;   // elements per lane

// DPP moves (row-local lane permutations, full rate, no LDS).
template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), CTRL, 0xF, 0xF, true));
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

template <int N>
__device__ __forceinline__ void load_f32(float (&dst)[N], const float* __restrict__ src) {
  static_assert(N % 4 == 0, "vector loads");
#pragma unroll
  for (int i = 0; i < N / 4; ++i) {
    const float4 t = reinterpret_cast<const float4*>(src)[i];
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

__device__ __forceinline__ uint32_t fbits(float x) { return __float_as_uint(x); }

// x & m, opaque to the optimiser: keeps "(w >> 8b) & 0xFF -> float" as one
// v_cvt_f32_ubyte<b> per element instead of a bit-field extract plus a convert.
__device__ __forceinline__ uint32_t and_opaque(uint32_t x, uint32_t m) {
  uint32_t r;
  asm("v_and_b32 %0, %1, %2" : "=v"(r) : "v"(x), "v"(m));
  return r;
}

// max of two rounded values by their bit patterns (as signed integers): the
// same order as the floats whenever one of them is >= 0, which always holds
// here; no NaN canonicalisation of the inputs is needed.
__device__ __forceinline__ float max_bits(float a, float b) {
  return __int_as_float(max(__float_as_int(a), __float_as_int(b)));
}

// d[i] = a[i] * b + c rounded toward +infinity (i = 0..7).  The single-
// precision rounding field of the MODE register is switched for exactly these
// eight instructions and restored to round-to-nearest-even.
__device__ __forceinline__ void fma_ru8(float* d, const float* a, float b, float c) {
  asm volatile(
      "s_setreg_imm32_b32 hwreg(HW_REG_MODE, 0, 2), 1\n\t"
      "s_nop 1\n\t"
      "v_fma_f32 %0, %8, %16, %17\n\t"
      "v_fma_f32 %1, %9, %16, %17\n\t"
      "v_fma_f32 %2, %10, %16, %17\n\t"
      "v_fma_f32 %3, %11, %16, %17\n\t"
      "v_fma_f32 %4, %12, %16, %17\n\t"
      "v_fma_f32 %5, %13, %16, %17\n\t"
      "v_fma_f32 %6, %14, %16, %17\n\t"
      "v_fma_f32 %7, %15, %16, %17\n\t"
      "s_nop 1\n\t"
      "s_setreg_imm32_b32 hwreg(HW_REG_MODE, 0, 2), 0"
      : "=&v"(d[0]), "=&v"(d[1]), "=&v"(d[2]), "=&v"(d[3]), "=&v"(d[4]), "=&v"(d[5]),
        "=&v"(d[6]), "=&v"(d[7])
      : "v"(a[0]), "v"(a[1]), "v"(a[2]), "v"(a[3]), "v"(a[4]), "v"(a[5]), "v"(a[6]), "v"(a[7]),
        "v"(b), "v"(c));
}

// Code format of a lane's 32 elements.
template <int BITS>
struct Fmt {
  static constexpr int NW = BITS == 4 ? 4 : 8;                  // 32-bit words per lane
  static constexpr uint32_t OFF = BITS == 4 ? 0x88888888u : 0x80808080u;  // two's compl. <-> offset
  static constexpr uint32_t ONES = BITS == 4 ? 0x11111111u : 0x01010101u;
  static constexpr uint32_t FIELD = BITS == 4 ? 0xFu : 0xFFu;
  static constexpr float BIAS = BITS == 4 ? 8.f : 128.f;        // offset code = C + BIAS
  static constexpr float QMAX = BITS == 4 ? 7.f : 127.f;
  static constexpr float MQ = kMagic + BIAS;                    // rounding constant, offset built in
};

// Offset-binary code words -> unsigned code values (element order = column order).
template <int BITS>
__device__ __forceinline__ void unpack_offsets(const uint32_t (&xo)[Fmt<BITS>::NW], float (&f)[EPL]) {
  if constexpr (BITS == 4) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint32_t lo = and_opaque(xo[j], 0x0F0F0F0Fu);          // even columns, one per byte
      const uint32_t hi = and_opaque(xo[j] >> 4, 0x0F0F0F0Fu);     // odd columns
      f[8 * j + 0] = static_cast<float>(lo & 0xFFu);
      f[8 * j + 1] = static_cast<float>(hi & 0xFFu);
      f[8 * j + 2] = static_cast<float>((lo >> 8) & 0xFFu);
      f[8 * j + 3] = static_cast<float>((hi >> 8) & 0xFFu);
      f[8 * j + 4] = static_cast<float>((lo >> 16) & 0xFFu);
      f[8 * j + 5] = static_cast<float>((hi >> 16) & 0xFFu);
      f[8 * j + 6] = static_cast<float>(lo >> 24);
      f[8 * j + 7] = static_cast<float>(hi >> 24);
    }
  } else {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      f[4 * j + 0] = static_cast<float>(xo[j] & 0xFFu);
      f[4 * j + 1] = static_cast<float>((xo[j] >> 8) & 0xFFu);
      f[4 * j + 2] = static_cast<float>((xo[j] >> 16) & 0xFFu);
      f[4 * j + 3] = static_cast<float>(xo[j] >> 24);
    }
  }
}

// Gather the low bytes of four words into one word.
__device__ __forceinline__ uint32_t gather_low_bytes(uint32_t a, uint32_t b, uint32_t c, uint32_t d) {
  const uint32_t ab = __builtin_amdgcn_perm(b, a, 0x0C0C0400u);   // [a0, b0, 0, 0]
  const uint32_t cd = __builtin_amdgcn_perm(d, c, 0x04000C0Cu);   // [0, 0, c0, d0]
  return ab | cd;
}

// Rounded values t (low byte = offset code, byte 1 zero) -> offset-binary words.
template <int BITS>
__device__ __forceinline__ void pack_offsets(const float (&t)[EPL], uint32_t (&X)[Fmt<BITS>::NW]) {
  if constexpr (BITS == 4) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      uint32_t p[4];
#pragma unroll
      for (int b = 0; b < 4; ++b) p[b] = (fbits(t[8 * j + 2 * b + 1]) << 4) | fbits(t[8 * j + 2 * b]);
      X[j] = gather_low_bytes(p[0], p[1], p[2], p[3]);
    }
  } else {
#pragma unroll
    for (int j = 0; j < 8; ++j)
      X[j] = gather_low_bytes(fbits(t[4 * j]), fbits(t[4 * j + 1]), fbits(t[4 * j + 2]),
                              fbits(t[4 * j + 3]));
  }
}

// Per-lane row data, loaded one iteration ahead.
template <int BITS>
struct RowIn {
  uint32_t x[Fmt<BITS>::NW];
  float s;
  float v;
};

template <int BITS, int DK>
__device__ __forceinline__ void load_row(RowIn<BITS>& R, const StepArgs& a, size_t row, int lc, int gi) {
  constexpr int ROWB = DK * BITS / 8;
  const uint8_t* p = a.codes + row * ROWB + lc * (EPL * BITS / 8);
#pragma unroll
  for (int c = 0; c < Fmt<BITS>::NW / 4; ++c) {
    const uint4 w = reinterpret_cast<const uint4*>(p)[c];
    R.x[4 * c + 0] = w.x;
    R.x[4 * c + 1] = w.y;
    R.x[4 * c + 2] = w.z;
    R.x[4 * c + 3] = w.w;
  }
  R.s = a.scales[row * a.ng + gi];
  R.v = a.v[row];
}

template <int BITS, int DK, int POLICY, int ROUND, int DELTA, int DIAG>
__global__ __launch_bounds__(256) void step_kernel(StepArgs a) {
  using F = Fmt<BITS>;
  constexpr int NW = F::NW;
  constexpr int LPR = DK / EPL;          // lanes per row
  constexpr int RPI = 64 / LPR;          // rows per wave-iteration
  constexpr int ROWB = DK * BITS / 8;    // packed bytes per row
  constexpr bool BDR = ROUND == RND_BDR;
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

  // Oriented frame for directional rounding: per column rho_c = sign(k_c)
  // (the sign bit, so -0 counts as negative).  Kf marks, nibble- or byte-wise,
  // the columns whose codes are negated.  A zero k_c has no update direction:
  // such a wave patches those elements out of the round-up candidate.
  uint32_t Kx[BDR ? NW : 1], K1[BDR ? NW : 1], Kf[BDR ? NW : 1];
  float qn[(BDR && POLICY == POL_YOKED) ? EPL : 4];
  bool kzero_wave = false;
  if constexpr (BDR) {
    bool kzero = false;
#pragma unroll
    for (int e = 0; e < EPL; ++e) kzero |= (kk[e] == 0.f);
    kzero_wave = __any(kzero);
    // v_perm selector 9 (11) replicates the sign bit of the second (first) operand
#pragma unroll
    for (int j = 0; j < NW; ++j) {
      uint32_t m;
      if constexpr (BITS == 8) {
        const float* kq = &kk[4 * j];
        m = __builtin_amdgcn_perm(fbits(kq[1]), fbits(kq[0]), 0x0C0C0B09u) |
            __builtin_amdgcn_perm(fbits(kq[3]), fbits(kq[2]), 0x0B090C0Cu);
      } else {
        const float* kq = &kk[8 * j];
        const uint32_t ev = __builtin_amdgcn_perm(fbits(kq[2]), fbits(kq[0]), 0x0C0C0B09u) |
                            __builtin_amdgcn_perm(fbits(kq[6]), fbits(kq[4]), 0x0B090C0Cu);
        const uint32_t od = __builtin_amdgcn_perm(fbits(kq[3]), fbits(kq[1]), 0x0C0C0B09u) |
                            __builtin_amdgcn_perm(fbits(kq[7]), fbits(kq[5]), 0x0B090C0Cu);
        m = (ev & 0x0F0F0F0Fu) | (od & 0xF0F0F0F0u);
      }
      Kf[j] = m;
      Kx[j] = m ^ F::OFF;
      K1[j] = m & F::ONES;
    }
#pragma unroll
    for (int e = 0; e < EPL; ++e) {
      if constexpr (POLICY == POL_YOKED) qn[e] = qq[e];
      qq[e] = __uint_as_float(fbits(qq[e]) ^ (fbits(kk[e]) & 0x80000000u));   // q oriented
    }
  }

  const int it0 = slice * a.nit;
  auto row_of = [&](int it, bool& live) {
    const int r = (it0 + it) * RPI + lr;
    live = r < a.dv;                     // uniform over the lanes of a row
    return (size_t)h * a.dv + (live ? r : a.dv - 1);
  };

  RowIn<BITS> nxt;
  bool live_n;
  size_t row_n = row_of(0, live_n);
  load_row<BITS, DK>(nxt, a, row_n, lc, gi);

  for (int it = 0; it < a.nit; ++it) {
    const RowIn<BITS> in = nxt;
    const bool live = live_n;
    const size_t row = row_n;
    if (it + 1 < a.nit) {
      row_n = row_of(it + 1, live_n);
      load_row<BITS, DK>(nxt, a, row_n, lc, gi);
    }
    float R[POLICY == POL_YOKED ? EPL : 4];
    float* rp = a.ref + row * DK + col0;
    if constexpr (POLICY == POL_YOKED) load_f32(R, rp);

    // dequantise (oriented for BDR): S' = fma(u, m, -bias*m) = fl(C * fl(s*alpha))
    uint32_t xo[NW];
#pragma unroll
    for (int j = 0; j < NW; ++j) {
      if constexpr (BDR)
        xo[j] = (in.x[j] ^ Kx[j]) + K1[j];   // offset code, negated where k_c < 0
      else
        xo[j] = in.x[j] ^ F::OFF;
    }
    float sp[EPL];
    unpack_offsets<BITS>(xo, sp);
    if constexpr (DIAG) {
#pragma unroll
      for (int e = 0; e < EPL; ++e) {
        const float m = in.s * aa[e];
        sp[e] = (sp[e] - F::BIAS) * m;
      }
    } else {
      const float m = in.s * alpha_s;
      const float mb = -F::BIAS * m;
#pragma unroll
      for (int e = 0; e < EPL; ++e) sp[e] = fmaf(sp[e], m, mb);
    }

    // delta correction u = S' . k and the write coefficient w = beta (v - u)
    float u = 0.f;
    if constexpr (DELTA) {
      float p = 0.f;
#pragma unroll
      for (int e = 0; e < EPL; ++e) p = fmaf(sp[e], BDR ? fabsf(kk[e]) : kk[e], p);
      u = row_sum<LPR>(p);
    }
    const float w = beta * (in.v - u);

    // rank-one write and readout o_r = S_t . q (before requantisation)
    float st[EPL];
    float po = 0.f;
#pragma unroll
    for (int e = 0; e < EPL; ++e) {
      st[e] = fmaf(w, BDR ? fabsf(kk[e]) : kk[e], sp[e]);
      po = fmaf(st[e], qq[e], po);
    }
    const float o = row_sum<LPR>(po);
    if (live && lc == 0) a.o[row] = o;

    // scale policy
    float snew = in.s;
    if constexpr (POLICY == POL_YOKED) {
      // advance the fp32 reference row with the same update (natural frame)
#pragma unroll
      for (int e = 0; e < EPL; ++e) R[e] = R[e] * (DIAG ? aa[e] : alpha_s);
      float ur = 0.f;
      if constexpr (DELTA) {
        float p = 0.f;
#pragma unroll
        for (int e = 0; e < EPL; ++e) p = fmaf(R[e], kk[e], p);
        ur = row_sum<LPR>(p);
      }
      const float wr = beta * (in.v - ur);
      float pr = 0.f, amax = 0.f;
#pragma unroll
      for (int e = 0; e < EPL; ++e) {
        R[e] = fmaf(wr, kk[e], R[e]);
        pr = fmaf(R[e], BDR ? qn[e] : qq[e], pr);
        amax = fmaxf(amax, fabsf(R[e]));
      }
      const float oref = row_sum<LPR>(pr);
      if (live) {
        store_f32(rp, R);
        if (lc == 0 && a.o_ref) a.o_ref[row] = oref;
      }
      snew = group_max(amax, gl) / F::QMAX;
    } else if constexpr (POLICY == POL_DYNAMIC) {
      float amax = 0.f;
#pragma unroll
      for (int e = 0; e < EPL; ++e) amax = fmaxf(amax, fabsf(st[e]));
      snew = group_max(amax, gl) / F::QMAX;
    }
    const float inv = (snew == 0.f) ? 0.f : 1.0f / snew;

    // requantise
    float t[EPL];
    uint32_t X[NW];
    if constexpr (BDR) {
      // orient by sign(w) through the sign of inv: every update now points up
      const uint32_t wsign = fbits(w) & 0x80000000u;
      const float inv_w = __uint_as_float(fbits(inv) ^ wsign);
      const float mu = (w == 0.f) ? 0.f : F::MQ;     // w = 0: no update, no direction
      float tu[EPL];
#pragma unroll
      for (int b = 0; b < EPL / 8; ++b) fma_ru8(&tu[8 * b], &sp[8 * b], inv_w, mu);
      if (kzero_wave) {   // k_c = 0: no update, so no directional candidate
#pragma unroll
        for (int e = 0; e < EPL; ++e) tu[e] = (kk[e] == 0.f) ? 0.f : tu[e];
      }
#pragma unroll
      for (int e = 0; e < EPL; ++e) {
        const float tz = fmaf(st[e], inv_w, F::MQ);   // round half even of z = S*inv
        t[e] = __builtin_amdgcn_fmed3f(max_bits(tz, tu[e]), F::MQ - F::QMAX, F::MQ + F::QMAX);
      }
      pack_offsets<BITS>(t, X);
      // undo the orientation: negate offset codes by sign(w), then by sign(k_c)
      const uint32_t Wm = static_cast<uint32_t>(static_cast<int32_t>(fbits(w)) >> 31);
      const uint32_t W1 = Wm & F::ONES;
#pragma unroll
      for (int j = 0; j < NW; ++j) X[j] = ((((X[j] ^ Wm) + W1) ^ Kf[j]) + K1[j]) ^ F::OFF;
    } else {
#pragma unroll
      for (int e = 0; e < EPL; ++e)
        t[e] = __builtin_amdgcn_fmed3f(fmaf(st[e], inv, F::MQ), F::MQ - F::QMAX, F::MQ + F::QMAX);
      pack_offsets<BITS>(t, X);
#pragma unroll
      for (int j = 0; j < NW; ++j) X[j] ^= F::OFF;
    }

    if (live) {
      uint8_t* p = a.codes + row * ROWB + lc * (EPL * BITS / 8);
#pragma unroll
      for (int c = 0; c < NW / 4; ++c)
        reinterpret_cast<uint4*>(p)[c] = make_uint4(X[4 * c], X[4 * c + 1], X[4 * c + 2], X[4 * c + 3]);
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
