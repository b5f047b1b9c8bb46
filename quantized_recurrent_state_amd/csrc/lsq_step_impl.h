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
// its loads of codes are consecutive in memory.  The head's vectors (k, q, a
// diagonal decay) are staged once per wave in LDS and read per row.  The two
// row dot products and the group absmax are reduced across the lanes of a row
// with DPP butterflies; no atomics, no inter-wave traffic.  Every step
// re-reads and re-writes the whole packed state from HBM; the next row's
// codes, scale and v are loaded while the current row is computed.
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
// element (none when the round-up candidate is known to lie in the code
// range: then one med3 does both).  The packed result is turned back by the
// same xor-add.
#pragma once

#include <hip/hip_fp16.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "lsq_internal.h"

namespace lsq {
namespace dev {

enum { POL_DYNAMIC = 1, POL_PERSISTENT = 2, POL_YOKED = 3 };
enum { RND_RNE = 0, RND_BDR = 1, RND_DITHER = 2 };

// Golden-ratio Weyl dither: 2^32 (sqrt(5)-1)/2, truncated.  The offset of
// sequence position i is frac(i * 0.618...) = ((i * kWeyl) mod 2^32) / 2^32,
// used with 23 bits: the float 1 + u is 0x3F800000 | (w >> 9), one v_alignbit.
constexpr uint32_t kWeyl = 0x9E3779B9u;

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

template <int N>
__device__ __forceinline__ void store_lds(float* dst, const float (&src)[N]) {
#pragma unroll
  for (int i = 0; i < N / 4; ++i)
    reinterpret_cast<float4*>(dst)[i] = make_float4(src[4 * i], src[4 * i + 1], src[4 * i + 2],
                                                    src[4 * i + 3]);
}

__device__ __forceinline__ uint32_t fbits(float x) { return __float_as_uint(x); }

// One or two consecutive floats (a lane's share of a staged vector).
template <int N>
__device__ __forceinline__ void load_cols(float (&d)[N], const float* __restrict__ src) {
  if constexpr (N == 2) {
    const float2 t = *reinterpret_cast<const float2*>(src);
    d[0] = t.x;
    d[1] = t.y;
  } else {
    d[0] = src[0];
  }
}
template <int N>
__device__ __forceinline__ void store_cols(float* dst, const float (&v)[N]) {
  if constexpr (N == 2)
    *reinterpret_cast<float2*>(dst) = make_float2(v[0], v[1]);
  else
    dst[0] = v[0];
}


// x & m, opaque to the optimiser: keeps "(w >> 8b) & 0xFF -> float" as one
// v_cvt_f32_ubyte<b> per element instead of a bit-field extract plus a convert.
__device__ __forceinline__ uint32_t and_opaque(uint32_t x, uint32_t m) {
  uint32_t r;
  asm("v_and_b32 %0, %1, %2" : "=v"(r) : "v"(x), "v"(m));
  return r;
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

// d[i] = d[i] * b0 + c (i = 0..15) and d[i] * b1 + c (i = 16..31), rounded toward
// +infinity, in place: the 32 round-up candidates of a lane's row under one
// switch of the MODE register's single-precision rounding field (the block-of-
// eight form switches four times per row).
__device__ __forceinline__ void fma_ru32(float* d, float b0, float b1, float c) {
  asm volatile(
      "s_setreg_imm32_b32 hwreg(HW_REG_MODE, 0, 2), 1\n\t"
      "s_nop 1\n\t"
      "v_fma_f32 %0, %0, %32, %34\n\t"
      "v_fma_f32 %1, %1, %32, %34\n\t"
      "v_fma_f32 %2, %2, %32, %34\n\t"
      "v_fma_f32 %3, %3, %32, %34\n\t"
      "v_fma_f32 %4, %4, %32, %34\n\t"
      "v_fma_f32 %5, %5, %32, %34\n\t"
      "v_fma_f32 %6, %6, %32, %34\n\t"
      "v_fma_f32 %7, %7, %32, %34\n\t"
      "v_fma_f32 %8, %8, %32, %34\n\t"
      "v_fma_f32 %9, %9, %32, %34\n\t"
      "v_fma_f32 %10, %10, %32, %34\n\t"
      "v_fma_f32 %11, %11, %32, %34\n\t"
      "v_fma_f32 %12, %12, %32, %34\n\t"
      "v_fma_f32 %13, %13, %32, %34\n\t"
      "v_fma_f32 %14, %14, %32, %34\n\t"
      "v_fma_f32 %15, %15, %32, %34\n\t"
      "v_fma_f32 %16, %16, %33, %34\n\t"
      "v_fma_f32 %17, %17, %33, %34\n\t"
      "v_fma_f32 %18, %18, %33, %34\n\t"
      "v_fma_f32 %19, %19, %33, %34\n\t"
      "v_fma_f32 %20, %20, %33, %34\n\t"
      "v_fma_f32 %21, %21, %33, %34\n\t"
      "v_fma_f32 %22, %22, %33, %34\n\t"
      "v_fma_f32 %23, %23, %33, %34\n\t"
      "v_fma_f32 %24, %24, %33, %34\n\t"
      "v_fma_f32 %25, %25, %33, %34\n\t"
      "v_fma_f32 %26, %26, %33, %34\n\t"
      "v_fma_f32 %27, %27, %33, %34\n\t"
      "v_fma_f32 %28, %28, %33, %34\n\t"
      "v_fma_f32 %29, %29, %33, %34\n\t"
      "v_fma_f32 %30, %30, %33, %34\n\t"
      "v_fma_f32 %31, %31, %33, %34\n\t"
      "s_nop 1\n\t"
      "s_setreg_imm32_b32 hwreg(HW_REG_MODE, 0, 2), 0"
      : "+v"(d[0]), "+v"(d[1]), "+v"(d[2]), "+v"(d[3]), "+v"(d[4]), "+v"(d[5]), "+v"(d[6]), "+v"(d[7]),
        "+v"(d[8]), "+v"(d[9]), "+v"(d[10]), "+v"(d[11]), "+v"(d[12]), "+v"(d[13]), "+v"(d[14]), "+v"(d[15]),
        "+v"(d[16]), "+v"(d[17]), "+v"(d[18]), "+v"(d[19]), "+v"(d[20]), "+v"(d[21]), "+v"(d[22]), "+v"(d[23]),
        "+v"(d[24]), "+v"(d[25]), "+v"(d[26]), "+v"(d[27]), "+v"(d[28]), "+v"(d[29]), "+v"(d[30]), "+v"(d[31])
      : "v"(b0), "v"(b1), "v"(c));
}

// d[i] = (a[i] * b + e[i]) + c, both operations rounded toward -infinity:
// with e = 1 + u and c = MQ - 1 this is MQ + floor(a*b + u) exactly (the
// first rounding keeps the floor, the second lands on the integer grid).
__device__ __forceinline__ void fma_add_rd8(float* d, const float* a, float b, const float* e, float c) {
  asm volatile(
      "s_setreg_imm32_b32 hwreg(HW_REG_MODE, 0, 2), 2\n\t"
      "s_nop 1\n\t"
      "v_fma_f32 %0, %8, %24, %16\n\t"
      "v_fma_f32 %1, %9, %24, %17\n\t"
      "v_fma_f32 %2, %10, %24, %18\n\t"
      "v_fma_f32 %3, %11, %24, %19\n\t"
      "v_fma_f32 %4, %12, %24, %20\n\t"
      "v_fma_f32 %5, %13, %24, %21\n\t"
      "v_fma_f32 %6, %14, %24, %22\n\t"
      "v_fma_f32 %7, %15, %24, %23\n\t"
      "v_add_f32 %0, %0, %25\n\t"
      "v_add_f32 %1, %1, %25\n\t"
      "v_add_f32 %2, %2, %25\n\t"
      "v_add_f32 %3, %3, %25\n\t"
      "v_add_f32 %4, %4, %25\n\t"
      "v_add_f32 %5, %5, %25\n\t"
      "v_add_f32 %6, %6, %25\n\t"
      "v_add_f32 %7, %7, %25\n\t"
      "s_nop 1\n\t"
      "s_setreg_imm32_b32 hwreg(HW_REG_MODE, 0, 2), 0"
      : "=&v"(d[0]), "=&v"(d[1]), "=&v"(d[2]), "=&v"(d[3]), "=&v"(d[4]), "=&v"(d[5]),
        "=&v"(d[6]), "=&v"(d[7])
      : "v"(a[0]), "v"(a[1]), "v"(a[2]), "v"(a[3]), "v"(a[4]), "v"(a[5]), "v"(a[6]), "v"(a[7]),
        "v"(e[0]), "v"(e[1]), "v"(e[2]), "v"(e[3]), "v"(e[4]), "v"(e[5]), "v"(e[6]), "v"(e[7]),
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

// Offset-binary code words -> unsigned code values (element order = column
// order), for one block of eight elements: wb holds its words (one INT4 word,
// two INT8 words).
template <int BITS>
__device__ __forceinline__ void unpack_block(const uint32_t* wb, float (&f)[8]) {
  if constexpr (BITS == 4) {
    const uint32_t lo = and_opaque(wb[0], 0x0F0F0F0Fu);          // even columns, one per byte
    const uint32_t hi = and_opaque(wb[0] >> 4, 0x0F0F0F0Fu);     // odd columns
    f[0] = static_cast<float>(lo & 0xFFu);
    f[1] = static_cast<float>(hi & 0xFFu);
    f[2] = static_cast<float>((lo >> 8) & 0xFFu);
    f[3] = static_cast<float>((hi >> 8) & 0xFFu);
    f[4] = static_cast<float>((lo >> 16) & 0xFFu);
    f[5] = static_cast<float>((hi >> 16) & 0xFFu);
    f[6] = static_cast<float>(lo >> 24);
    f[7] = static_cast<float>(hi >> 24);
  } else {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const uint32_t x = wb[h];
      f[4 * h + 0] = static_cast<float>(x & 0xFFu);
      f[4 * h + 1] = static_cast<float>((x >> 8) & 0xFFu);
      f[4 * h + 2] = static_cast<float>((x >> 16) & 0xFFu);
      f[4 * h + 3] = static_cast<float>(x >> 24);
    }
  }
}

template <int BITS>
__device__ __forceinline__ void unpack_offsets(const uint32_t (&xo)[Fmt<BITS>::NW], float (&f)[EPL]) {
#pragma unroll
  for (int b = 0; b < EPL / 8; ++b) {
    float t[8];
    unpack_block<BITS>(&xo[b * (BITS == 4 ? 1 : 2)], t);
#pragma unroll
    for (int i = 0; i < 8; ++i) f[8 * b + i] = t[i];
  }
}

// a * b + c with a the low (HI = false) or high half of h taken as binary16,
// b and c binary32, one rounding to binary32 (v_fma_mix_f32).  An offset code
// u placed in the low bits of a half is the binary16 subnormal u * 2^-24,
// converted exactly (binary16 subnormals are kept by the kernel's float mode).
template <bool HI>
__device__ __forceinline__ float fma_mix(uint32_t h, float b, float c) {
  float d;
  if constexpr (HI)
    asm("v_fma_mix_f32 %0, %1, %2, %3 op_sel:[1,0,0] op_sel_hi:[1,0,0]" : "=v"(d) : "v"(h), "v"(b), "v"(c));
  else
    asm("v_fma_mix_f32 %0, %1, %2, %3 op_sel:[0,0,0] op_sel_hi:[1,0,0]" : "=v"(d) : "v"(h), "v"(b), "v"(c));
  return d;
}

// Offset-binary code words -> S' = fl(C * m) = fl(u * m - bias * m), without
// a separate int -> float conversion: two codes at a time are masked into the
// low bits of the two halves of a word (binary16 subnormals u * 2^-24, or
// 16u * 2^-24 for INT4 high nibbles) and v_fma_mix_f32 multiplies them by
// m * 2^24 (resp. m * 2^20), both exact scalings of m.  One block of eight
// elements (wb: its words) with the block's multiplier m and bias product mb.
template <int BITS>
__device__ __forceinline__ void dequant_mix_block(const uint32_t* wb, float m, float mb,
                                                  float (&f)[8]) {
  if constexpr (BITS == 4) {
    const float m24 = m * 0x1p24f, m20 = m * 0x1p20f;
    const uint32_t x = wb[0];
    const uint32_t a = x & 0x000F000Fu;          // columns 8b, 8b+4
    const uint32_t bb = x & 0x00F000F0u;         // columns 8b+1, 8b+5 (times 16)
    const uint32_t c = (x >> 8) & 0x000F000Fu;   // columns 8b+2, 8b+6
    const uint32_t d = (x >> 8) & 0x00F000F0u;   // columns 8b+3, 8b+7 (times 16)
    f[0] = fma_mix<false>(a, m24, mb);
    f[4] = fma_mix<true>(a, m24, mb);
    f[1] = fma_mix<false>(bb, m20, mb);
    f[5] = fma_mix<true>(bb, m20, mb);
    f[2] = fma_mix<false>(c, m24, mb);
    f[6] = fma_mix<true>(c, m24, mb);
    f[3] = fma_mix<false>(d, m20, mb);
    f[7] = fma_mix<true>(d, m20, mb);
  } else {
    const float m24 = m * 0x1p24f;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const uint32_t x = wb[h];
      const uint32_t a = x & 0x00FF00FFu;                         // columns 4j, 4j+2
      const uint32_t c = __builtin_amdgcn_perm(x, x, 0x0C030C01u);  // columns 4j+1, 4j+3
      f[4 * h + 0] = fma_mix<false>(a, m24, mb);
      f[4 * h + 2] = fma_mix<true>(a, m24, mb);
      f[4 * h + 1] = fma_mix<false>(c, m24, mb);
      f[4 * h + 3] = fma_mix<true>(c, m24, mb);
    }
  }
}

// All 32 elements of a lane.  With two groups per lane (GPL = 2, 16-element
// groups) elements 0-15 take m[0] and elements 16-31 m[1].
template <int BITS, int GPL>
__device__ __forceinline__ void dequant_mix(const uint32_t (&xo)[Fmt<BITS>::NW], const float (&mm)[GPL],
                                            const float (&mbb)[GPL], float (&f)[EPL]) {
#pragma unroll
  for (int b = 0; b < EPL / 8; ++b) {
    float t[8];
    dequant_mix_block<BITS>(&xo[b * (BITS == 4 ? 1 : 2)], mm[GPL == 2 ? b / 2 : 0],
                            mbb[GPL == 2 ? b / 2 : 0], t);
#pragma unroll
    for (int i = 0; i < 8; ++i) f[8 * b + i] = t[i];
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

// Eight rounded values (elements 8b..8b+7) -> the offset-binary word(s) they fill.
template <int BITS>
__device__ __forceinline__ void pack_block(const float (&t)[8], uint32_t* X) {
  if constexpr (BITS == 4) {
    uint32_t p[4];
#pragma unroll
    for (int b = 0; b < 4; ++b) p[b] = (fbits(t[2 * b + 1]) << 4) | fbits(t[2 * b]);
    X[0] = gather_low_bytes(p[0], p[1], p[2], p[3]);
  } else {
    X[0] = gather_low_bytes(fbits(t[0]), fbits(t[1]), fbits(t[2]), fbits(t[3]));
    X[1] = gather_low_bytes(fbits(t[4]), fbits(t[5]), fbits(t[6]), fbits(t[7]));
  }
}

// 16-byte accesses of the packed codes.  Every state byte is written once per
// step and not read again within it, so the stores carry the non-temporal
// hint (the nt bit), which speeds up a read-then-write stream on gfx950.  The
// loads carry it too (NTL) when the state is far larger than the last-level
// cache: a head's span then streams as fast as a copy of it; on a state the
// Infinity Cache holds between steps the hint would send the next step to
// HBM, so those launches keep default loads.
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
template <bool NTL = false>
__device__ __forceinline__ u32x4 load_codes16(const uint8_t* p) {
  if constexpr (NTL)
    return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
  else
    return *reinterpret_cast<const u32x4*>(p);
}
__device__ __forceinline__ void store_codes16(uint8_t* p, u32x4 v) {
  __builtin_nontemporal_store(v, reinterpret_cast<u32x4*>(p));
}

// Per-lane row data, loaded one iteration ahead.
// Stored group-scale formats.  A 16-bit scale converts to fp32 exactly; an
// fp32 scale is rounded to the stored format to nearest, ties to even
// (binary16 by the conversion instruction in the default rounding mode, with
// subnormals; bfloat16 by rounding the discarded 16 bits of the pattern).
enum { SFMT_F32 = 0, SFMT_F16 = 1, SFMT_BF16 = 2 };

__device__ __forceinline__ float scale_from16(uint32_t bits16, int sfmt) {
  return sfmt == SFMT_F16 ? __half2float(__ushort_as_half((unsigned short)bits16))
                          : __uint_as_float(bits16 << 16);
}

__device__ __forceinline__ uint32_t scale_to16(float s, int sfmt) {
  if (sfmt == SFMT_F16) return __half_as_ushort(__float2half_rn(s));
  const uint32_t u = __float_as_uint(s);             // finite, non-negative
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

template <int BITS, int GPL>
struct RowIn {
  uint32_t x[Fmt<BITS>::NW];
  float s[GPL];       // the lane's group scale(s)
  uint32_t sw;        // 16-bit scale pattern(s) as loaded, converted just before use
  float v;
};

// Wave-uniform bases of one head's rows (scalar registers); a lane adds a
// 32-bit offset, so per-row addressing costs a few VALU ops.
struct HeadPtrs {
  uint8_t* codes;
  float* scales;
  const float* v;
  float* o;
  float* o_ref;
  float* ref;
};

// Element of a head array at a 32-bit byte offset (a wave-uniform base in
// scalar registers plus one VGPR: the global_load/store "saddr" form).
template <typename T>
__device__ __forceinline__ T& at_bytes(T* base, uint32_t byte_off) {
  return *reinterpret_cast<T*>(reinterpret_cast<char*>(base) + byte_off);
}
template <typename T>
__device__ __forceinline__ const T& at_bytes(const T* base, uint32_t byte_off) {
  return *reinterpret_cast<const T*>(reinterpret_cast<const char*>(base) + byte_off);
}

template <int BITS, int DK, int GPL, bool NTL = false>
__device__ __forceinline__ void load_row(RowIn<BITS, GPL>& R, const HeadPtrs& H, int ng, uint32_t r,
                                         int lc, int gi, int sfmt = SFMT_F32) {
  constexpr int ROWB = DK * BITS / 8;
  const uint8_t* p = H.codes + (r * ROWB + lc * (EPL * BITS / 8));
#pragma unroll
  for (int c = 0; c < Fmt<BITS>::NW / 4; ++c) {
    const u32x4 w = load_codes16<NTL>(p + 16 * c);
    R.x[4 * c + 0] = w.x;
    R.x[4 * c + 1] = w.y;
    R.x[4 * c + 2] = w.z;
    R.x[4 * c + 3] = w.w;
  }
  if (sfmt == SFMT_F32) {
    if constexpr (GPL == 2) {
      const float2 s2 = at_bytes(reinterpret_cast<const float2*>(H.scales), (r * ng + gi) * 4u);
      R.s[0] = s2.x;
      R.s[1] = s2.y;
    } else {
      R.s[0] = at_bytes(H.scales, (r * ng + gi) * 4u);
    }
  } else if constexpr (GPL == 2) {       // both 16-bit scales in one dword
    R.sw = at_bytes(reinterpret_cast<const uint32_t*>(H.scales), (r * ng + gi) * 2u);
  } else {
    R.sw = at_bytes(reinterpret_cast<const uint16_t*>(H.scales), (r * ng + gi) * 2u);
  }
  R.v = at_bytes(H.v, r * 4u);
}

// 16-bit scales of a prefetched row to fp32, right before the row is used (a
// conversion next to the load would wait for it).
template <int BITS, int GPL>
__device__ __forceinline__ void resolve_scales(RowIn<BITS, GPL>& R, int sfmt) {
  if (sfmt == SFMT_F32) return;
  if constexpr (GPL == 2) {
    R.s[0] = scale_from16(R.sw & 0xFFFFu, sfmt);
    R.s[1] = scale_from16(R.sw >> 16, sfmt);
  } else {
    R.s[0] = scale_from16(R.sw, sfmt);
  }
}

// fl(1/s): v_rcp_f32 followed by one fma Newton step reproduces the correctly
// rounded reciprocal for every s in [2^-126, 2^126) on gfx950 (all 2^31
// positive floats compared with IEEE division; it differs only where s or
// 1/s is subnormal).  0 and out-of-range scales take the IEEE division.
__device__ __forceinline__ float inv_scale(float s) {
  const float r0 = __builtin_amdgcn_rcpf(s);
  const float e = fmaf(-s, r0, 1.0f);
  float r = fmaf(e, r0, r0);
  if (__builtin_expect(!(s >= 0x1p-126f && s < 0x1p126f), 0)) r = (s == 0.f) ? 0.f : 1.0f / s;
  return r;
}

#ifndef LSQ_STEP_WAVES_PER_EU
#define LSQ_STEP_WAVES_PER_EU 2
#endif

// Per-lane, per-head state of a wave: its place in the grid, the orientation
// masks of its 32 columns, and where the head's vectors sit in LDS.  The
// vectors (k, q, a diagonal decay; oriented for directional rounding) are
// staged once per wave in LDS (3 KiB per wave at most) and read per row,
// which keeps them out of the register file: more waves fit on a SIMD.
constexpr int kVecs = 5;   // k, q, alpha, natural k, natural q
// Orientation masks of INT8 codes (three times eight words per lane) live in
// LDS when a row takes two passes (the delta rule, or a scale computed from
// the updated row), which hold S' or S for the whole row; the one-pass linear
// write under a frozen scale has registers to spare and keeps them in
// registers (fewer LDS reads per row: the directional rounding of the INT8
// Mamba-2-style workload runs within 5% of round-to-nearest that way, against
// 20% with the masks in LDS).  INT4's twelve words always stay in registers.
template <int BITS, int DK, int ROUND, int DELTA, int POLICY>
struct LdsPlan {
  static constexpr int NW = Fmt<BITS>::NW;
  static constexpr int LPR = DK / EPL;
  static constexpr bool ONE_PASS = !DELTA && POLICY == POL_PERSISTENT;
  static constexpr bool MASKS = ROUND == RND_BDR && BITS == 8 && !ONE_PASS;
  static constexpr int MASK_WORDS = MASKS ? 3 * NW * LPR : 0;   // Kf, Kx, K1 per column chunk
  // Each vector is stored as LPR chunks of 32 floats, one per column chunk of
  // a row, PAD floats apart: the chunks a wave's lanes read together (four at
  // Dk = 128) then start in different LDS banks instead of all in bank 0.
  static constexpr int PAD = 4;
  static constexpr int CHUNK = EPL + PAD;
  static constexpr int VSTRIDE = LPR * CHUNK;     // floats per staged vector
  static constexpr int WAVE_FLOATS = kVecs * VSTRIDE + MASK_WORDS;
};
template <int BITS, int DK, int POLICY, int ROUND, int DELTA, int DIAG>
struct Lane {
  static constexpr bool BDR = ROUND == RND_BDR;
  static constexpr int NW = Fmt<BITS>::NW;
  static constexpr bool REG_MASKS = BDR && !LdsPlan<BITS, DK, ROUND, DELTA, POLICY>::MASKS;
  int h, slice, lr, lc, col0, gl, gi;
  int vbase;          // float offset of this wave's vectors in the LDS array
  HeadPtrs H;         // this head's rows
  float alpha_s, beta;
  float alpha_hi;     // max |alpha_c| over the head (the scalar decay's |alpha|)
  // max |alpha_c| <= 1 - 2^-20: then fl(qmax fl(s |alpha_c|)) fl(1/s) < qmax for
  // every zero or normal scale s (three roundings of relative size <= 2^-22
  // cannot make up a 2^-20 deficit, subnormal intermediates included), so the
  // per-row test of the round-up candidate's range is known to pass
  bool decay_in_range;
  uint32_t Kf[REG_MASKS ? NW : 1], Kx[REG_MASKS ? NW : 1], K1[REG_MASKS ? NW : 1];
};

// Eight consecutive floats of an LDS vector, read with two 16-byte loads.
// The row loop passes a base offset laundered through an empty asm once per
// row, so that these reads stay inside the loop instead of being hoisted into
// registers; the block offsets are constants (immediate ds_read offsets).
template <int DK>
__device__ __forceinline__ void lds_block(float (&d)[8], const float* lds, int off) {
  const float4 a = *reinterpret_cast<const float4*>(lds + off);
  const float4 b = *reinterpret_cast<const float4*>(lds + off + 4);
  d[0] = a.x; d[1] = a.y; d[2] = a.z; d[3] = a.w;
  d[4] = b.x; d[5] = b.y; d[6] = b.z; d[7] = b.w;
}
template <int N>
__device__ __forceinline__ void lds_words(uint32_t (&d)[N], const float* lds, int off) {
#pragma unroll
  for (int i = 0; i < N / 4; ++i) {
    const uint4 t = *reinterpret_cast<const uint4*>(lds + off + 4 * i);
    d[4 * i] = t.x; d[4 * i + 1] = t.y; d[4 * i + 2] = t.z; d[4 * i + 3] = t.w;
  }
}

// The row loop of one wave.  KZ: the head's key has a zero component (no
// update direction there), so those elements drop their round-up candidate.
template <int BITS, int DK, int POLICY, int ROUND, int DELTA, int DIAG, int GPL, int SF, bool KZ,
          bool NTL, bool PRE>
__device__ __forceinline__ void row_loop(const StepArgs& a, Lane<BITS, DK, POLICY, ROUND, DELTA, DIAG>& L,
                                         const float* vec, RowIn<BITS, GPL>& bufA, bool liveA,
                                         uint32_t rowA) {
  // stored scale format, fixed per instance (SFMT_*): the other formats'
  // paths are compiled out
  constexpr int sfmt = SF;
  using P = LdsPlan<BITS, DK, ROUND, DELTA, POLICY>;
  // vec + L.vbase + v*VSTRIDE + L.lc*CHUNK: this lane's 32 columns of vector v
  const int base0 = L.vbase + L.lc * P::CHUNK;
  // vec + mbase0 + m*LPR*NW: this lane's words of mask m (Kf, Kx, K1)
  const int mbase0 = L.vbase + kVecs * P::VSTRIDE + L.lc * P::NW;
  using F = Fmt<BITS>;
  constexpr int NW = F::NW;
  constexpr int LPR = DK / EPL;          // lanes per row
  constexpr int RPI = 64 / LPR;          // rows per wave-iteration
  constexpr int ROWB = DK * BITS / 8;    // packed bytes per row
  constexpr int WPB = BITS == 4 ? 1 : 2; // code words per block of 8 elements
  constexpr bool BDR = ROUND == RND_BDR;

  const int it0 = L.slice * a.nit;
  const HeadPtrs& H = L.H;
  auto row_of = [&](int it, bool& live) -> uint32_t {
    const int r = (it0 + it) * RPI + L.lr;
    live = r < a.dv;                     // uniform over the lanes of a row
    return (uint32_t)min(r, a.dv - 1);
  };

  // One row, from dequantisation to the packed store.
  auto process = [&](const RowIn<BITS, GPL>& in, const bool live, const uint32_t row) {

    int base = base0;
    asm volatile("" : "+v"(base));
    int mbase = mbase0;
    if constexpr (P::MASKS) asm volatile("" : "+v"(mbase));
    // words j0 .. j0+N-1 of orientation mask m (0: Kf, 1: Kx, 2: K1)
    auto mask = [&](int m, int j0, auto& d) {
      constexpr int N = sizeof(d) / sizeof(d[0]);
      if constexpr (P::MASKS) {
        if constexpr (N % 4 == 0) {
          lds_words<N>(d, vec, mbase + m * LPR * NW + j0);
        } else {
#pragma unroll
          for (int j = 0; j < N; ++j)
            d[j] = reinterpret_cast<const uint32_t*>(vec)[mbase + m * LPR * NW + j0 + j];
        }
      } else if constexpr (BDR) {
#pragma unroll
        for (int j = 0; j < N; ++j)
          d[j] = m == 0 ? L.Kf[j0 + j] : (m == 1 ? L.Kx[j0 + j] : L.K1[j0 + j]);
      }
    };
    (void)mask;
    const int kOff = base, qOff = base + P::VSTRIDE, aOff = base + 2 * P::VSTRIDE;
    const int knOff = base + 3 * P::VSTRIDE, qnOff = base + 4 * P::VSTRIDE;
    (void)qOff; (void)aOff; (void)knOff; (void)qnOff;
    float R[POLICY == POL_YOKED ? EPL : 4];
    float* rp = &at_bytes(H.ref, (row * DK + L.col0) * 4u);
    if constexpr (POLICY == POL_YOKED) load_f32(R, rp);

    // Linear write under a frozen scale: w, the scale and the reciprocal are
    // known before any element, so each block of eight is dequantised,
    // written, read out and rounded in one pass and neither S' nor S is held
    // for the whole row (fewer registers, more waves per SIMD).
    constexpr bool ONE_PASS = P::ONE_PASS;
    // dequantise (oriented for BDR): S' = fma(u, m, -bias*m) = fl(C * fl(s*alpha));
    // offset codes of words j0 .. j0+N-1, negated where k_c < 0 (BDR)
    auto orient = [&](int j0, auto& d) {
      constexpr int N = sizeof(d) / sizeof(d[0]);
      if constexpr (BDR) {
        uint32_t kx[N], k1[N];
        mask(1, j0, kx);
        mask(2, j0, k1);
#pragma unroll
        for (int j = 0; j < N; ++j) d[j] = (in.x[j0 + j] ^ kx[j]) + k1[j];
      } else {
#pragma unroll
        for (int j = 0; j < N; ++j) d[j] = in.x[j0 + j] ^ F::OFF;
      }
    };
    uint32_t xo[ONE_PASS ? 1 : NW];
    if constexpr (!ONE_PASS) orient(0, xo);
    float m[GPL], mb[GPL];
#pragma unroll
    for (int h = 0; h < GPL; ++h) {
      m[h] = in.s[h] * L.alpha_s;
      mb[h] = -F::BIAS * m[h];
    }
    // S' of the block of eight elements 8b .. 8b+7
    auto dequant_block = [&](int b, float (&f)[8]) {
      uint32_t wl[WPB];
      const uint32_t* wb = &xo[ONE_PASS ? 0 : WPB * b];
      if constexpr (ONE_PASS) {
        orient(WPB * b, wl);
        wb = wl;
      }
      if constexpr (DIAG) {
        unpack_block<BITS>(wb, f);
        float ab[8];
        lds_block<DK>(ab, vec, aOff + 8 * b);
#pragma unroll
        for (int i = 0; i < 8; ++i) f[i] = (f[i] - F::BIAS) * (in.s[GPL == 2 ? b / 2 : 0] * ab[i]);
      } else {
        dequant_mix_block<BITS>(wb, m[GPL == 2 ? b / 2 : 0], mb[GPL == 2 ? b / 2 : 0], f);
      }
    };
    float sp[ONE_PASS ? 1 : EPL];
    if constexpr (!ONE_PASS) {
#pragma unroll
      for (int b = 0; b < EPL / 8; ++b) {
        float t[8];
        dequant_block(b, t);
#pragma unroll
        for (int i = 0; i < 8; ++i) sp[8 * b + i] = t[i];
      }
    }

    // delta correction u = S' . k and the write coefficient w = beta (v - u)
    float u = 0.f;
    if constexpr (DELTA) {
      float p = 0.f;
#pragma unroll
      for (int b = 0; b < EPL / 8; ++b) {
        float kb[8];
        lds_block<DK>(kb, vec, kOff + 8 * b);
#pragma unroll
        for (int i = 0; i < 8; ++i) p = fmaf(sp[8 * b + i], kb[i], p);
      }
      u = row_sum<LPR>(p);
    }
    const float w = L.beta * (in.v - u);

    uint32_t X[NW];
    // Orientation by sign(w) (directional rounding), for w < 0: the rounding
    // runs on -S and -S' (inv and the rounding constant negated), so a rounded
    // value is -(MQ + c) with c the code in the key-oriented frame; its low
    // mantissa bits, which the packing takes, are those of MQ + c, and the
    // clamp bounds are negated with it.  w = 0 (of either sign) has no
    // direction and is not negated.
    const uint32_t wsign = (BDR && w < 0.f) ? 0x80000000u : 0u;
    const float mq_w = __uint_as_float(fbits(F::MQ) ^ wsign);          // +-MQ
    const float top_w = mq_w + F::QMAX, bot_w = mq_w - F::QMAX;         // the clamp, negated with it
    const float mu = (w == 0.f) ? 0.f : mq_w;
    // back from the key-oriented frame: negate offset codes where k_c < 0
    auto unorient = [&](uint32_t x, uint32_t kf, uint32_t k1) -> uint32_t {
      if constexpr (BDR)
        return ((x ^ kf) + k1) ^ F::OFF;
      else
        return x ^ F::OFF;
    };
    // Weyl sequence position of this lane's first element of the row
    const uint32_t dbase = a.dither_base + row * a.dither_row + (uint32_t)L.col0 * kWeyl;
    (void)dbase;
    // round one block of eight: S (and S' for BDR) -> offset codes
    // IN_RANGE: every ceil(z') of the row lies in [-qmax, qmax], so that
    // clamp(max(tz, tu)) = med3(tz, tu, MQ + qmax), one instruction.
    auto round_block = [&](auto in_range, const float* stb, const float* spb, float inv, int b) {
      constexpr bool IN_RANGE = decltype(in_range)::value;
      float t[8];
      if constexpr (BDR) {
        const float inv_w = __uint_as_float(fbits(inv) ^ wsign);
        float tu[8];
        if constexpr (ONE_PASS) {
          fma_ru8(tu, spb, inv_w, mu);                 // ceil(z') + MQ
        } else {
#pragma unroll
          for (int i = 0; i < 8; ++i) tu[i] = spb[i];  // already ceil(z') + MQ (fma_ru32)
        }
        if constexpr (KZ) {
          // no update direction where k_c = 0: the candidate is the clamp's floor
          float kb[8];
          lds_block<DK>(kb, vec, kOff + 8 * b);
#pragma unroll
          for (int i = 0; i < 8; ++i) tu[i] = (kb[i] == 0.f) ? bot_w : tu[i];
        }
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const float tz = fmaf(stb[i], inv_w, mq_w);   // +-(MQ + round half even of z)
          if constexpr (IN_RANGE)
            t[i] = __builtin_amdgcn_fmed3f(tz, tu[i], top_w);
          else
            t[i] = __builtin_amdgcn_fmed3f(__builtin_amdgcn_fmed3f(tz, tu[i], __builtin_inff()), bot_w,
                                           top_w);   // max(tz, tu), then the clamp
        }
      } else if constexpr (ROUND == RND_DITHER) {
        // floor(z + u) with the Weyl offsets of elements 8b .. 8b+7
        float e[8];
#pragma unroll
        for (int i = 0; i < 8; ++i)   // ({0x7F, w} >> 9) = 0x3F800000 | (w >> 9): the float 1 + u
          e[i] = __uint_as_float(__builtin_amdgcn_alignbit(0x7Fu, dbase + (uint32_t)(8 * b + i) * kWeyl, 9));
        fma_add_rd8(t, stb, inv, e, F::MQ - 1.f);
#pragma unroll
        for (int i = 0; i < 8; ++i) t[i] = __builtin_amdgcn_fmed3f(t[i], F::MQ - F::QMAX, F::MQ + F::QMAX);
      } else {
#pragma unroll
        for (int i = 0; i < 8; ++i)
          t[i] = __builtin_amdgcn_fmed3f(fmaf(stb[i], inv, F::MQ), F::MQ - F::QMAX, F::MQ + F::QMAX);
      }
      uint32_t xb[WPB], kf[WPB], k1[WPB];
      pack_block<BITS>(t, xb);
      if constexpr (BDR) {
        mask(0, WPB * b, kf);
        mask(2, WPB * b, k1);
      }
#pragma unroll
      for (int i = 0; i < WPB; ++i) X[WPB * b + i] = unorient(xb[i], kf[i], k1[i]);
    };

    float snew[GPL];
    uint32_t s16[GPL] = {};
#pragma unroll
    for (int h = 0; h < GPL; ++h) snew[h] = in.s[h];
    float po = 0.f;
    if constexpr (ONE_PASS) {
      float inv[GPL];
#pragma unroll
      for (int h = 0; h < GPL; ++h) inv[h] = inv_scale(snew[h]);
      bool in_range = false;
      if constexpr (BDR) {
        in_range = L.decay_in_range;
        if (!in_range) {
          bool ok = true;
#pragma unroll
          for (int h = 0; h < GPL; ++h) {
            const float mq = F::QMAX * fabsf(in.s[h] * L.alpha_hi);
            ok = ok && fmaf(mq, inv[h], -F::QMAX) <= 0.f;
          }
          in_range = __all(ok);
        }
      }
      auto pass = [&](auto in_range_t) {
#pragma unroll
        for (int b = 0; b < EPL / 8; ++b) {
          float spb[8], stb[8], kb[8], qb[8];
          dequant_block(b, spb);
          lds_block<DK>(kb, vec, kOff + 8 * b);
          lds_block<DK>(qb, vec, qOff + 8 * b);
#pragma unroll
          for (int i = 0; i < 8; ++i) {
            stb[i] = fmaf(w, kb[i], spb[i]);
            po = fmaf(stb[i], qb[i], po);
          }
          round_block(in_range_t, stb, spb, inv[GPL == 2 ? b / 2 : 0], b);
        }
      };
      if (in_range)
        pass(std::true_type{});
      else
        pass(std::false_type{});
      const float o = row_sum<LPR>(po);
      if (live && L.lc == 0) at_bytes(H.o, row * 4u) = o;
    } else {
      // rank-one write and readout o_r = S_t . q (before requantisation)
      float st[EPL];
#pragma unroll
      for (int b = 0; b < EPL / 8; ++b) {
        float kb[8], qb[8];
        lds_block<DK>(kb, vec, kOff + 8 * b);
        lds_block<DK>(qb, vec, qOff + 8 * b);
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          st[8 * b + i] = fmaf(w, kb[i], sp[8 * b + i]);
          po = fmaf(st[8 * b + i], qb[i], po);
        }
      }
      const float o = row_sum<LPR>(po);
      if (live && L.lc == 0) at_bytes(H.o, row * 4u) = o;
      float amax[GPL] = {};
      if constexpr (POLICY == POL_YOKED) {
        // advance the fp32 reference row with the same update (natural frame)
        const int krOff = BDR ? knOff : kOff, qrOff = BDR ? qnOff : qOff;
#pragma unroll
        for (int b = 0; b < EPL / 8; ++b) {
          float ab[8];
          if constexpr (DIAG) lds_block<DK>(ab, vec, aOff + 8 * b);
#pragma unroll
          for (int i = 0; i < 8; ++i) R[8 * b + i] = R[8 * b + i] * (DIAG ? ab[i] : L.alpha_s);
        }
        float ur = 0.f;
        if constexpr (DELTA) {
          float p = 0.f;
#pragma unroll
          for (int b = 0; b < EPL / 8; ++b) {
            float kb[8];
            lds_block<DK>(kb, vec, krOff + 8 * b);
#pragma unroll
            for (int i = 0; i < 8; ++i) p = fmaf(R[8 * b + i], kb[i], p);
          }
          ur = row_sum<LPR>(p);
        }
        const float wr = L.beta * (in.v - ur);
        float pr = 0.f;
#pragma unroll
        for (int b = 0; b < EPL / 8; ++b) {
          float kb[8], qb[8];
          lds_block<DK>(kb, vec, krOff + 8 * b);
          lds_block<DK>(qb, vec, qrOff + 8 * b);
#pragma unroll
          for (int i = 0; i < 8; ++i) {
            const int e = 8 * b + i;
            R[e] = fmaf(wr, kb[i], R[e]);
            pr = fmaf(R[e], qb[i], pr);
            amax[GPL == 2 ? e / 16 : 0] = fmaxf(amax[GPL == 2 ? e / 16 : 0], fabsf(R[e]));
          }
        }
        const float oref = row_sum<LPR>(pr);
        if (live) {
          store_f32(rp, R);
          if (L.lc == 0 && H.o_ref) at_bytes(H.o_ref, row * 4u) = oref;
        }
      } else if constexpr (POLICY == POL_DYNAMIC) {
#pragma unroll
        for (int e = 0; e < EPL; ++e)
          amax[GPL == 2 ? e / 16 : 0] = fmaxf(amax[GPL == 2 ? e / 16 : 0], fabsf(st[e]));
      }
      if constexpr (POLICY != POL_PERSISTENT) {
        if constexpr (GPL == 2) {
          snew[0] = amax[0] / F::QMAX;               // groups inside the lane
          snew[1] = amax[1] / F::QMAX;
        } else {
          snew[0] = group_max(amax[0], L.gl) / F::QMAX;
        }
        if (sfmt != SFMT_F32) {            // the stored value forms the codes
#pragma unroll
          for (int h = 0; h < GPL; ++h) {
            s16[h] = scale_to16(snew[h], sfmt);
            snew[h] = scale_from16(s16[h], sfmt);
          }
        }
      }
      float inv[GPL];
#pragma unroll
      for (int h = 0; h < GPL; ++h) inv[h] = inv_scale(snew[h]);
      // With an unchanged scale, |z'| = |S'| inv <= fl(qmax fl(s |alpha|)) inv;
      // when that bound is <= qmax on every lane (any decay with |alpha| below
      // one by a few ulps), the round-up candidate needs no clamp of its own.
      // w = 0 (mu = 0) leaves tu = ceil(z') below the clamp's floor and tz
      // within it, so the median is min(tz, MQ + qmax) there as well.
      bool in_range = false;
      if constexpr (BDR && POLICY == POL_PERSISTENT) {
        in_range = L.decay_in_range;
        if (!in_range) {
          bool ok = true;
#pragma unroll
          for (int h = 0; h < GPL; ++h) {
            const float mq = F::QMAX * fabsf(in.s[h] * L.alpha_hi);
            ok = ok && fmaf(mq, inv[h], -F::QMAX) <= 0.f;
          }
          in_range = __all(ok);
        }
      }
      if constexpr (BDR) {   // the row's round-up candidates, in place of S'
        fma_ru32(sp, __uint_as_float(fbits(inv[0]) ^ wsign),
                 __uint_as_float(fbits(inv[GPL - 1]) ^ wsign), mu);
      }
      if (in_range) {
#pragma unroll
        for (int b = 0; b < EPL / 8; ++b)
          round_block(std::true_type{}, &st[8 * b], &sp[8 * b], inv[GPL == 2 ? b / 2 : 0], b);
      } else {
#pragma unroll
        for (int b = 0; b < EPL / 8; ++b)
          round_block(std::false_type{}, &st[8 * b], &sp[8 * b], inv[GPL == 2 ? b / 2 : 0], b);
      }
    }

    if (live) {
      uint8_t* p = H.codes + (row * ROWB + L.lc * (EPL * BITS / 8));
#pragma unroll
      for (int c = 0; c < NW / 4; ++c)
        store_codes16(p + 16 * c, u32x4{X[4 * c], X[4 * c + 1], X[4 * c + 2], X[4 * c + 3]});
      if constexpr (POLICY != POL_PERSISTENT) {
        if (sfmt == SFMT_F32) {
          if constexpr (GPL == 2)
            at_bytes(reinterpret_cast<float2*>(H.scales), (row * a.ng + L.gi) * 4u) =
                make_float2(snew[0], snew[1]);
          else if ((L.lc % L.gl) == 0)
            at_bytes(H.scales, (row * a.ng + L.gi) * 4u) = snew[0];
        } else if constexpr (GPL == 2) {
          at_bytes(reinterpret_cast<uint32_t*>(H.scales), (row * a.ng + L.gi) * 2u) =
              s16[0] | (s16[1] << 16);
        } else if ((L.lc % L.gl) == 0) {
          at_bytes(reinterpret_cast<uint16_t*>(H.scales), (row * a.ng + L.gi) * 2u) = (uint16_t)s16[0];
        }
      }
    }
  };

  // Rows in pairs with two prefetch buffers (no register copies between rows).
  // PRE: the caller has requested the first row (bufA, liveA, rowA) already
  if constexpr (!PRE) {
    rowA = row_of(0, liveA);
    load_row<BITS, DK, GPL, NTL>(bufA, H, a.ng, rowA, L.lc, L.gi, sfmt);
  }
  RowIn<BITS, GPL> bufB;
  bool liveB;
  uint32_t rowB = 0;
  for (int it = 0; it < a.nit; it += 2) {
    if (it + 1 < a.nit) {
      rowB = row_of(it + 1, liveB);
      load_row<BITS, DK, GPL, NTL>(bufB, H, a.ng, rowB, L.lc, L.gi, sfmt);
    }
    resolve_scales(bufA, sfmt);
    process(bufA, liveA, rowA);
    if (it + 1 >= a.nit) break;
    if (it + 2 < a.nit) {
      rowA = row_of(it + 2, liveA);
      load_row<BITS, DK, GPL, NTL>(bufA, H, a.ng, rowA, L.lc, L.gi, sfmt);
    }
    resolve_scales(bufB, sfmt);
    process(bufB, liveB, rowB);
  }
}

template <int BITS, int DK, int POLICY, int ROUND, int DELTA, int DIAG, int GPL, int SF,
          bool NTL = false>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(LSQ_STEP_WAVES_PER_EU)))
void step_kernel(StepArgs a) {
  using F = Fmt<BITS>;
  constexpr int NW = F::NW;
  constexpr int LPR = DK / EPL;
  constexpr bool BDR = ROUND == RND_BDR;
  static_assert(LPR >= 1 && LPR <= 16, "row must fit a 16-lane DPP row");

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(blockIdx.x * 4 + (threadIdx.x >> 6));
  if (wave >= a.total_waves) return;     // whole waves only
  Lane<BITS, DK, POLICY, ROUND, DELTA, DIAG> L;
  using P = LdsPlan<BITS, DK, ROUND, DELTA, POLICY>;
  L.h = wave / a.waves_per_head;
  L.slice = wave - L.h * a.waves_per_head;
  {
    const size_t row0 = (size_t)L.h * a.dv;
    L.H.codes = a.codes + row0 * (DK * BITS / 8);
    L.H.scales = reinterpret_cast<float*>(reinterpret_cast<char*>(a.scales) +
                                          row0 * a.ng * (SF ? 2 : 4));
    if (a.head_scale) L.H.scales = a.scales + L.h;   // one frozen scale per head (ng = 0)
    L.H.v = a.v + row0;
    L.H.o = a.o + row0;
    L.H.o_ref = a.o_ref ? a.o_ref + row0 : nullptr;
    L.H.ref = a.ref ? a.ref + row0 * DK : nullptr;
  }
  L.lr = lane / LPR;
  L.lc = lane % LPR;
  L.col0 = L.lc * EPL;
  L.gl = a.group / EPL;                  // lanes per group (>= 1)
  L.gi = L.col0 / a.group;               // this lane's group

  // per-head vectors for this lane's columns (staged in LDS below)
  __shared__ float4 vec4[4 * P::WAVE_FLOATS / 4];
  float* vec = reinterpret_cast<float*>(vec4);
  L.vbase = (threadIdx.x >> 6) * P::WAVE_FLOATS;
  // The head's vectors are staged by all 64 lanes, DK/64 columns each: a
  // lane loads, transforms and stores only its own columns (sc, sc+1), at
  // their place in the padded chunk layout.  Directional rounding also needs
  // the sign bits of the lane's own 32 row columns (kk) for its orientation
  // masks.
  constexpr int CPL = DK / 64;
  static_assert(CPL == 1 || CPL == 2, "staging takes one or two columns per lane");
  const int sc = lane * CPL;
  const int soff = L.vbase + (sc / EPL) * P::CHUNK + (sc % EPL);
  float ks[CPL], qs[CPL];
  load_cols<CPL>(ks, a.k + (size_t)L.h * DK + sc);
  load_cols<CPL>(qs, a.q + (size_t)L.h * DK + sc);
  float kk[BDR ? EPL : 4];
  if constexpr (BDR) load_f32(kk, a.k + (size_t)L.h * DK + L.col0);
  // The wave's first row (codes, scale, v) is requested before the head's
  // vectors arrive, so that the two loads' latencies overlap, except in the
  // persistent-BDR instances where holding that row through the set-up below
  // would take the kernel past 128 VGPRs (below four waves per SIMD): INT8 with
  // the delta rule or two groups per lane, INT4 with the delta rule and two
  // groups per lane or a diagonal decay.  Those request it after the set-up.
  constexpr bool HOIST = !(POLICY == POL_PERSISTENT && BDR &&
                           (BITS == 8 ? (DELTA || GPL == 2) : (DELTA && (GPL == 2 || DIAG))));
  RowIn<BITS, GPL> row0in;
  bool live0 = false;
  uint32_t row0 = 0;
  if constexpr (HOIST) {
    constexpr int RPI = 64 / LPR;
    const int r = L.slice * a.nit * RPI + L.lr;
    live0 = r < a.dv;
    row0 = (uint32_t)min(r, a.dv - 1);
    load_row<BITS, DK, GPL, NTL>(row0in, L.H, a.ng, row0, L.lc, L.gi, SF);
  }
  L.alpha_s = DIAG ? 1.f : a.alpha[L.h];
  L.alpha_hi = fabsf(L.alpha_s);
  L.beta = a.beta[L.h];
  const bool writer = L.lr == 0;         // one lane per column chunk fills the INT8 masks
  if constexpr (DIAG) {
    float as[CPL];
    load_cols<CPL>(as, a.alpha + (size_t)L.h * DK + sc);
    store_cols<CPL>(vec + soff + 2 * P::VSTRIDE, as);
    float am = fabsf(as[0]);
    if constexpr (CPL == 2) am = fmaxf(am, fabsf(as[1]));
    am = group_max(am, 16);                              // within each 16-lane row
    am = fmaxf(am, __shfl_xor(am, 16));
    L.alpha_hi = fmaxf(am, __shfl_xor(am, 32));          // over the head's DK columns
  }

  L.decay_in_range = __builtin_amdgcn_readfirstlane(L.alpha_hi <= 0x1.ffffep-1f ? 1 : 0) != 0;

  bool kzero = false;
  if constexpr (BDR) {
#pragma unroll
    for (int i = 0; i < CPL; ++i) kzero |= (ks[i] == 0.f);
    // Oriented frame: per column rho_c = sign(k_c) (the sign bit, so -0 counts
    // as negative).  Kf marks, nibble- or byte-wise, the negated columns.
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
      if constexpr (P::MASKS) {
        if (writer) {
          float* mp = vec + L.vbase + kVecs * P::VSTRIDE + L.lc * NW;
          reinterpret_cast<uint32_t*>(mp)[j] = m;
          reinterpret_cast<uint32_t*>(mp + LPR * NW)[j] = m ^ F::OFF;
          reinterpret_cast<uint32_t*>(mp + 2 * LPR * NW)[j] = m & F::ONES;
        }
      } else {
        L.Kf[j] = m;
        L.Kx[j] = m ^ F::OFF;
        L.K1[j] = m & F::ONES;
      }
    }
    if constexpr (POLICY == POL_YOKED) {
      store_cols<CPL>(vec + soff + 3 * P::VSTRIDE, ks);
      store_cols<CPL>(vec + soff + 4 * P::VSTRIDE, qs);
    }
#pragma unroll
    for (int i = 0; i < CPL; ++i) {
      qs[i] = __uint_as_float(fbits(qs[i]) ^ (fbits(ks[i]) & 0x80000000u));
      ks[i] = fabsf(ks[i]);
    }
  }
  store_cols<CPL>(vec + soff + 0 * P::VSTRIDE, ks);
  store_cols<CPL>(vec + soff + 1 * P::VSTRIDE, qs);
  // LDS accesses of one wave execute in order; the barrier keeps the compiler
  // from moving reads of the staged vectors above these writes.
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

  if constexpr (BDR) {
    if (__any(kzero))
      row_loop<BITS, DK, POLICY, ROUND, DELTA, DIAG, GPL, SF, true, NTL, HOIST>(a, L, vec, row0in, live0, row0);
    else
      row_loop<BITS, DK, POLICY, ROUND, DELTA, DIAG, GPL, SF, false, NTL, HOIST>(a, L, vec, row0in, live0, row0);
  } else {
    row_loop<BITS, DK, POLICY, ROUND, DELTA, DIAG, GPL, SF, false, NTL, HOIST>(a, L, vec, row0in, live0, row0);
  }
}

// Dispatch one (BITS, DK) family over the method flags and the group size
// (16-element groups: two groups per lane; 32 and more: one).
template <int BITS, int DK, int SF>
hipError_t launch_family(const StepArgs& a, int policy, int rounding, int delta, int diag,
                         hipStream_t s) {
  static_assert(SF == SFMT_F32 || SF == SFMT_F16 || SF == SFMT_BF16, "stored scale format");
  const dim3 grid((a.total_waves + 3) / 4), block(256);
  const int gpl = a.group < EPL ? 2 : 1;   // 16-element groups: two per lane
  // non-temporal code loads for states far larger than the last-level cache,
  // instantiated for the INT4 frozen-scale, scalar-decay, 32-or-more-element-
  // group instances with fp32 scales and RNE or directional rounding (the long
  // multi-layer decode: 2% faster there; the INT8 launch of the same stack
  // measured slower with them)
  constexpr bool NT_FAMILY = SF == SFMT_F32 && BITS == 4;
#define LSQ_CASE(P, R, D, G)                                                                       \
  if (policy == P && rounding == R && delta == D && diag == G) {                                   \
    if (gpl == 2)                                                                                  \
      hipLaunchKernelGGL((step_kernel<BITS, DK, P, R, D, G, 2, SF>), grid, block, 0, s, a);        \
    else if (NT_FAMILY && P == POL_PERSISTENT && G == 0 && R != RND_DITHER && a.nt_loads)          \
      hipLaunchKernelGGL((step_kernel<BITS, DK, P, R, D, G, 1, SF, NT_FAMILY && P == POL_PERSISTENT && G == 0 && R != RND_DITHER>), \
                         grid, block, 0, s, a);                                                    \
    else                                                                                           \
      hipLaunchKernelGGL((step_kernel<BITS, DK, P, R, D, G, 1, SF>), grid, block, 0, s, a);        \
    return hipGetLastError();                                                                      \
  }
#define LSQ_CASES_PR(P, R) \
  LSQ_CASE(P, R, 0, 0) LSQ_CASE(P, R, 0, 1) LSQ_CASE(P, R, 1, 0) LSQ_CASE(P, R, 1, 1)
#define LSQ_CASES_P(P) LSQ_CASES_PR(P, RND_RNE) LSQ_CASES_PR(P, RND_BDR) LSQ_CASES_PR(P, RND_DITHER)
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
