// Chunkwise prefill state pass (linear write, delta = 0) on the matrix cores.
//
// "LinQuant: Functional Invariances for Low-Precision Linear Recurrences"
// (summary page), Methodology, Low-Precision Chunkwise Realization: per chunk
// of C tokens the state write H = Q(B V)^T Q(Gamma-> (.) K) and the state pass
// S_[i+1] = Q(gamma^C S_[i] + H).  Reading (the oracle's): Gamma->_t is the
// fp32 suffix product of the chunk's later decays, gamma^C the chunk's
// product; B V = fl(beta v); one INT8 absmax scale per operand block (head,
// chunk); the integer product is exact, H = fl(h fl(s_V s_K)); X = fma(gamma,
// S, H) requantised in the state's group format and policy (RNE; a dynamic
// scale is rounded to the stored scale format, fp32, binary16 or bfloat16,
// before the codes are formed); S carried as fl(code s).
//
// One workgroup of eight waves per head walks the chunks in order, as a
// three-stage pipeline with one barrier per chunk.  Waves 0-3 build operands,
// waves 4-7 own the state; each SIMD runs one of each, so the operand waves'
// memory waits hide behind the state waves' arithmetic and back.  In
// iteration i:
//   operand waves  (a) quantise the operand columns of chunk i+1, held in
//                  registers since the previous iteration, with the block
//                  absmax the waves posted then; INT8 codes go to LDS
//                  transposed ([column][token], rows padded to 72 bytes),
//                  double-buffered;
//                  (b) read chunk i+2: thread c < Dk builds column c of
//                  Gamma-> (.) K (its decay suffix product in the oracle's
//                  order), thread 128 + i column i of B V, 64 tokens each in
//                  registers, and posts its wave's absmax;
//   state waves    H of chunk i on v_mfma_i32_16x16x32_i8 with A = K codes
//                  (rows = state columns) and B = V codes (columns = state
//                  rows), so lane l holds four adjacent columns 16I + 4(l/16)
//                  + v of state row 16J + l%16; then the state pass on the
//                  codes kept in LDS: group absmax in-lane, over the group's
//                  tiles and over the four lanes holding the row.
// The packed state is read into LDS at the start and written back at the end.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "lsq_step_impl.h"

namespace lsq {
namespace dev {

constexpr int kChunk = 64;
constexpr int kOpRow = 72;          // bytes per LDS operand row (64 tokens + pad)
typedef int i32x4 __attribute__((ext_vector_type(4)));

// Two's-complement INT8 code of x * inv rounded half to even, clamped to
// +-qmax (the magic constant without offset leaves the code in the low byte).
__device__ __forceinline__ int rne_code(float x, float inv, float qmax) {
  const float t = __builtin_amdgcn_fmed3f(fmaf(x, inv, kMagic), kMagic - qmax, kMagic + qmax);
  return (int)(__float_as_uint(t) - __float_as_uint(kMagic));
}

__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x = fmaxf(x, __shfl_xor(x, o));
  return x;
}

// S16: the state's scales are stored in a 16-bit format (a.sfmt picks
// binary16 or bfloat16); the fp32 instances carry no conversion code.
// HEAD: one scale per head (group 0).  A dynamic head scale needs the absmax
// of the whole head's X before any code is formed: the four state waves post
// their maxima to LDS and meet at one more barrier per chunk, which the
// operand waves also take, so that both roles count the same barriers.
template <int BITS, int DK, int DV, int POLICY, int DIAG, bool S16, bool HEAD>
__global__ __launch_bounds__(512) void prefill_kernel(PrefillArgs a) {
  constexpr float QMAX = BITS == 4 ? 7.f : 127.f;
  constexpr int RT = DV / 64;            // 16-row tiles per state wave
  constexpr int CT = DK / 16;            // 16-column tiles
  constexpr int ROWB = DK * BITS / 8;    // packed bytes per state row
  constexpr int SP = DK + 8;             // LDS pitch of a state code row (bank spread)
  constexpr int KW = DK / 64, VW = DV / 64;   // operand waves per side
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int h = blockIdx.x;
  const int ng = a.ng, g = a.group;
  const int nchunk = (a.T + kChunk - 1) / kChunk;

  __shared__ __align__(16) int8_t vt[2][DV * kOpRow];   // (B V)^T codes [dv][token]
  __shared__ __align__(16) int8_t kt[2][DK * kOpRow];   // (Gamma-> K)^T codes [dk][token]
  __shared__ __align__(16) int8_t stage[DV * SP];       // state codes [dv][dk]
  __shared__ float sscale[DV * 8];                      // state scales [dv][ng] (ng <= 8)
  __shared__ __align__(16) float gam[2][DK];            // gamma^C per column
  __shared__ float wmax[2][4];                          // per operand wave block absmax
  __shared__ float opscale[2][2];                       // s_V, s_K
  __shared__ float hmax[4];                             // per state wave |X| max (HEAD)
  constexpr bool XB = HEAD && POLICY == POL_DYNAMIC;    // the extra barrier per chunk

  // ---- the head's packed state -> LDS codes and scales.  The state stays
  // there as codes between chunks: the carried value is fl(code * scale).
  const size_t hrow0 = (size_t)h * DV;
  const uint32_t* gcodes = reinterpret_cast<const uint32_t*>(a.codes + hrow0 * ROWB);
  for (int idx = tid; idx < DV * ROWB / 4; idx += 512) {
    const int r = idx / (ROWB / 4), w = idx % (ROWB / 4);
    const uint32_t word = gcodes[idx];
    if constexpr (BITS == 4) {           // 8 nibbles -> 8 sign-extended bytes
      uint32_t lo = 0, hi = 0;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        lo |= (uint32_t)((((word >> (4 * q)) & 0xF) ^ 8) - 8) << (8 * q) & (0xFFu << (8 * q));
        hi |= (uint32_t)((((word >> (4 * q + 16)) & 0xF) ^ 8) - 8) << (8 * q) & (0xFFu << (8 * q));
      }
      *reinterpret_cast<uint32_t*>(&stage[r * SP + 8 * w]) = lo;
      *reinterpret_cast<uint32_t*>(&stage[r * SP + 8 * w + 4]) = hi;
    } else {
      *reinterpret_cast<uint32_t*>(&stage[r * SP + 4 * w]) = word;
    }
  }
  // scales as the fp32 values they represent (a 16-bit scale converts exactly)
  const uint16_t* scales16 = reinterpret_cast<const uint16_t*>(a.scales);
  if constexpr (HEAD) {
    if (tid == 0) sscale[0] = S16 ? scale_from16(scales16[h], a.sfmt) : a.scales[h];
  } else {
    for (int idx = tid; idx < DV * ng; idx += 512)
      sscale[idx] = S16 ? scale_from16(scales16[hrow0 * ng + idx], a.sfmt) : a.scales[hrow0 * ng + idx];
  }

  const int64_t nh = a.n_heads;
  const bool krole = wave < KW, vrole = wave >= 2 && wave < 2 + VW;
  const bool swave = wave >= 4;
  const unsigned ut = threadIdx.x;       // unsigned lane offset: scalar base + vector offset loads
  float col[kChunk];                     // operand column of the chunk in flight
  float gh = 1.f;                        // its gamma^C (K side)

  // Both roles run nchunk + 2 iterations with one barrier each, in two
  // separate loops (wave-uniform branch) so that neither holds the other's
  // registers.
  if (!swave) {
    for (int i = -2; i < nchunk; ++i) {
      // ---- (a) quantise chunk i+1's columns with the posted block maxima
      const int q = i + 1;
      if (q >= 0 && q < nchunk && (krole || vrole)) {
        const int slot = q & 1;
        float mk = wmax[slot][0], mv = wmax[slot][2];
        if (KW > 1) mk = fmaxf(mk, wmax[slot][1]);
        if (VW > 1) mv = fmaxf(mv, wmax[slot][3]);
        const float s_v = mv / 127.f, s_k = mk / 127.f;
        const float inv = inv_scale(krole ? s_k : s_v);
        int8_t* dst = krole ? &kt[slot][tid * kOpRow] : &vt[slot][(tid - 128) * kOpRow];
#pragma unroll
        for (int t4 = 0; t4 < kChunk / 4; ++t4) {
          uint32_t w = 0;
#pragma unroll
          for (int b = 0; b < 4; ++b) w |= (uint32_t)(rne_code(col[4 * t4 + b], inv, 127.f) & 0xFF) << (8 * b);
          reinterpret_cast<uint32_t*>(dst)[t4] = w;
        }
        if (krole) gam[slot][tid] = gh;
        if (tid == 0) {
          opscale[slot][0] = s_v;
          opscale[slot][1] = s_k;
        }
      }
      // ---- (b) read chunk i+2 and build its operand columns
      const int p = i + 2;
      if (p < nchunk && (krole || vrole)) {
        const int c0 = p * kChunk;
        const int tc = min(kChunk, a.T - c0);
        const int64_t row0 = (int64_t)c0 * nh + h;
        float v0[kChunk], v1[kChunk];
        float pl = 0.f;                  // per-token scalar (scalar decay, beta): lane t holds token t
        {
          const float* r0 = krole ? a.k + row0 * DK : a.v + row0 * DV - 128;
          const int64_t s0 = krole ? nh * DK : nh * DV;
          if (tc == kChunk) {            // full chunk: row pointers advance by one token
            const float* r = r0;
#pragma unroll
            for (int t = 0; t < kChunk; ++t, r += s0) v0[t] = r[ut];
          } else {                       // a short chunk re-reads its last token
#pragma unroll
            for (int t = 0; t < kChunk; ++t) v0[t] = r0[min(t, tc - 1) * s0 + ut];
          }
          if (krole && DIAG) {
            const float* ra = a.alpha + row0 * DK;
            if (tc == kChunk) {
              const float* r = ra;
#pragma unroll
              for (int t = 0; t < kChunk; ++t, r += nh * DK) v1[t] = r[ut];
            } else {
#pragma unroll
              for (int t = 0; t < kChunk; ++t) v1[t] = ra[min(t, tc - 1) * nh * DK + ut];
            }
          } else {
            const float* rs = krole ? a.alpha : a.beta;
            pl = rs[row0 + (int64_t)min(lane, tc - 1) * nh];
          }
        }
        float cmax = 0.f;
        if (krole) {
          float acc = 1.f;               // Gamma->: product of the later tokens' decays
#pragma unroll
          for (int t = kChunk - 1; t >= 0; --t) {
            const bool in = t < tc;
            const float dec =
                DIAG ? v1[t] : __int_as_float(__builtin_amdgcn_readlane(__float_as_int(pl), t));
            col[t] = in ? acc * v0[t] : 0.f;
            acc = in ? acc * dec : acc;
            cmax = fmaxf(cmax, fabsf(col[t]));
          }
          gh = acc;
        } else {
#pragma unroll
          for (int t = 0; t < kChunk; ++t) {
            const float b = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(pl), t));
            col[t] = t < tc ? b * v0[t] : 0.f;
            cmax = fmaxf(cmax, fabsf(col[t]));
          }
        }
        cmax = wave_max(cmax);
        if (lane == 0) wmax[p & 1][wave] = cmax;
      }
      if constexpr (XB) __syncthreads();   // the state waves' head maximum
      __syncthreads();
    }
  } else {
    __syncthreads();                     // iterations -2 and -1: operands only
    __syncthreads();
    if constexpr (XB) {
      __syncthreads();
      __syncthreads();
    }
    const int sw = wave - 4;
    for (int i = 0; i < nchunk; ++i) {
      const int slot = i & 1;
      const float s_v = opscale[slot][0], s_k = opscale[slot][1];
      // ---- H on the matrix cores
      i32x4 acc[RT][CT];
#pragma unroll
      for (int J = 0; J < RT; ++J)
#pragma unroll
        for (int I = 0; I < CT; ++I) acc[J][I] = i32x4{0, 0, 0, 0};
#pragma unroll
      for (int ks = 0; ks < kChunk / 32; ++ks) {
        const int koff = 32 * ks + 8 * (lane / 16);
        long bv[RT];
#pragma unroll
        for (int J = 0; J < RT; ++J)
          bv[J] = *reinterpret_cast<const long*>(&vt[slot][(16 * (sw * RT + J) + lane % 16) * kOpRow + koff]);
#pragma unroll
        for (int I = 0; I < CT; ++I) {
          const long ak = *reinterpret_cast<const long*>(&kt[slot][(16 * I + lane % 16) * kOpRow + koff]);
#pragma unroll
          for (int J = 0; J < RT; ++J)
            acc[J][I] = __builtin_amdgcn_mfma_i32_16x16x32_i8(ak, bv[J], acc[J][I], 0, 0, 0);
        }
      }
      // ---- state pass: X = fma(gamma, S, H), requantised per group
      const float sc = s_v * s_k;
      if constexpr (HEAD) {
        // one scale per head: X of both row tiles first, then the head's
        // absmax (dynamic), then the codes
        float x[RT][CT][4];
        float lmax = 0.f;
        const float s_old = sscale[0];
#pragma unroll
        for (int J = 0; J < RT; ++J) {
          const int r = 16 * (sw * RT + J) + lane % 16;
          const int8_t* crow = &stage[r * SP + 4 * (lane / 16)];
#pragma unroll
          for (int I = 0; I < CT; ++I) {
            float gc[4];
            if constexpr (DIAG) {
              const float4 q4 = *reinterpret_cast<const float4*>(&gam[slot][16 * I + 4 * (lane / 16)]);
              gc[0] = q4.x; gc[1] = q4.y; gc[2] = q4.z; gc[3] = q4.w;
            } else {
#pragma unroll
              for (int v = 0; v < 4; ++v) gc[v] = gam[slot][0];
            }
            const uint32_t cw = *reinterpret_cast<const uint32_t*>(&crow[16 * I]);
#pragma unroll
            for (int v = 0; v < 4; ++v) {
              const float S = (float)(int)(int8_t)(cw >> (8 * v)) * s_old;
              x[J][I][v] = fmaf(gc[v], S, (float)acc[J][I][v] * sc);
              lmax = fmaxf(lmax, fabsf(x[J][I][v]));
            }
          }
        }
        float sh = s_old;
        if constexpr (XB) {
          lmax = wave_max(lmax);
          if (lane == 0) hmax[sw] = lmax;
          __syncthreads();               // every state wave has read the old scale
          sh = fmaxf(fmaxf(hmax[0], hmax[1]), fmaxf(hmax[2], hmax[3])) / QMAX;
          if constexpr (S16) sh = scale_from16(scale_to16(sh, a.sfmt), a.sfmt);
          if (sw == 0 && lane == 0) sscale[0] = sh;
        }
        const float inv = inv_scale(sh);
#pragma unroll
        for (int J = 0; J < RT; ++J) {
          const int r = 16 * (sw * RT + J) + lane % 16;
          int8_t* crow = &stage[r * SP + 4 * (lane / 16)];
#pragma unroll
          for (int I = 0; I < CT; ++I) {
            uint32_t nw = 0;
#pragma unroll
            for (int v = 0; v < 4; ++v) nw |= (uint32_t)(rne_code(x[J][I][v], inv, QMAX) & 0xFF) << (8 * v);
            *reinterpret_cast<uint32_t*>(&crow[16 * I]) = nw;
          }
        }
        __syncthreads();
        continue;
      }
      const int tpg = g / 16;            // tiles per group (an aligned power of two)
#pragma unroll
      for (int J = 0; J < RT; ++J) {
        const int r = 16 * (sw * RT + J) + lane % 16;
        int8_t* crow = &stage[r * SP + 4 * (lane / 16)];
        float x[CT][4], s[CT];
#pragma unroll
        for (int I = 0; I < CT; ++I) {
          float gc[4];
          if constexpr (DIAG) {
            const float4 q4 = *reinterpret_cast<const float4*>(&gam[slot][16 * I + 4 * (lane / 16)]);
            gc[0] = q4.x; gc[1] = q4.y; gc[2] = q4.z; gc[3] = q4.w;
          } else {
#pragma unroll
            for (int v = 0; v < 4; ++v) gc[v] = gam[slot][0];
          }
          const uint32_t cw = *reinterpret_cast<const uint32_t*>(&crow[16 * I]);
          s[I] = sscale[r * ng + (16 * I) / g];
#pragma unroll
          for (int v = 0; v < 4; ++v) {
            const float S = (float)(int)(int8_t)(cw >> (8 * v)) * s[I];
            x[I][v] = fmaf(gc[v], S, (float)acc[J][I][v] * sc);
          }
        }
        if constexpr (POLICY == POL_DYNAMIC) {
          // group absmax: the tile's four columns in the lane, the group's
          // tiles by butterflies (static indices), then the four lanes that
          // hold the row (l%16 fixed)
          float m[CT];
#pragma unroll
          for (int I = 0; I < CT; ++I)
            m[I] = fmaxf(fmaxf(fabsf(x[I][0]), fabsf(x[I][1])), fmaxf(fabsf(x[I][2]), fabsf(x[I][3])));
#pragma unroll
          for (int step = 1; step < CT; step *= 2) {
            if (step < tpg) {
              float n2[CT];
#pragma unroll
              for (int I = 0; I < CT; ++I) n2[I] = fmaxf(m[I], m[I ^ step]);
#pragma unroll
              for (int I = 0; I < CT; ++I) m[I] = n2[I];
            }
          }
#pragma unroll
          for (int I = 0; I < CT; ++I) {
            m[I] = fmaxf(m[I], __shfl_xor(m[I], 16));
            m[I] = fmaxf(m[I], __shfl_xor(m[I], 32));
            s[I] = m[I] / QMAX;
            // a 16-bit format: the stored value forms the codes
            if constexpr (S16) s[I] = scale_from16(scale_to16(s[I], a.sfmt), a.sfmt);
            if (lane < 16 && (I % tpg) == 0) sscale[r * ng + (16 * I) / g] = s[I];
          }
        }
#pragma unroll
        for (int I = 0; I < CT; ++I) {
          const float inv = inv_scale(s[I]);
          uint32_t nw = 0;
#pragma unroll
          for (int v = 0; v < 4; ++v) nw |= (uint32_t)(rne_code(x[I][v], inv, QMAX) & 0xFF) << (8 * v);
          *reinterpret_cast<uint32_t*>(&crow[16 * I]) = nw;
        }
      }
      __syncthreads();
    }
  }
  if (nchunk == 0) return;
  // ---- LDS codes and scales -> the head's packed state
  uint32_t* ocodes = reinterpret_cast<uint32_t*>(a.codes + hrow0 * ROWB);
  for (int idx = tid; idx < DV * ROWB / 4; idx += 512) {
    const int r = idx / (ROWB / 4), w = idx % (ROWB / 4);
    uint32_t word;
    if constexpr (BITS == 4) {           // 8 bytes -> 8 nibbles
      const uint32_t lo = *reinterpret_cast<const uint32_t*>(&stage[r * SP + 8 * w]);
      const uint32_t hi = *reinterpret_cast<const uint32_t*>(&stage[r * SP + 8 * w + 4]);
      word = 0;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        word |= ((lo >> (8 * q)) & 0xF) << (4 * q);
        word |= ((hi >> (8 * q)) & 0xF) << (4 * q + 16);
      }
    } else {
      word = *reinterpret_cast<const uint32_t*>(&stage[r * SP + 4 * w]);
    }
    ocodes[idx] = word;
  }
  if constexpr (POLICY == POL_DYNAMIC && HEAD) {
    if (tid == 0) {
      if constexpr (S16)
        reinterpret_cast<uint16_t*>(a.scales)[h] = (uint16_t)scale_to16(sscale[0], a.sfmt);
      else
        a.scales[h] = sscale[0];
    }
  } else if constexpr (POLICY == POL_DYNAMIC) {
    uint16_t* out16 = reinterpret_cast<uint16_t*>(a.scales);
    for (int idx = tid; idx < DV * ng; idx += 512) {
      if constexpr (S16)   // already a value of the format: the conversion is exact
        out16[hrow0 * ng + idx] = (uint16_t)scale_to16(sscale[idx], a.sfmt);
      else
        a.scales[hrow0 * ng + idx] = sscale[idx];
    }
  }
}

}  // namespace dev

hipError_t launch_prefill(const PrefillArgs& a, int bits, int dk, int dv, int policy, int diag,
                          hipStream_t s) {
  const dim3 grid(a.n_heads), block(512);
#define LSQ_PF(B, DK, DV, P, G)                                                                   \
  if (bits == B && dk == DK && dv == DV && policy == P && diag == G) {                           \
    const bool s16 = a.sfmt != dev::SFMT_F32, head = a.group == 0;                               \
    if (!s16 && !head)                                                                           \
      hipLaunchKernelGGL((dev::prefill_kernel<B, DK, DV, P, G, false, false>), grid, block, 0, s, a); \
    else if (s16 && !head)                                                                       \
      hipLaunchKernelGGL((dev::prefill_kernel<B, DK, DV, P, G, true, false>), grid, block, 0, s, a); \
    else if (!s16)                                                                               \
      hipLaunchKernelGGL((dev::prefill_kernel<B, DK, DV, P, G, false, true>), grid, block, 0, s, a); \
    else                                                                                         \
      hipLaunchKernelGGL((dev::prefill_kernel<B, DK, DV, P, G, true, true>), grid, block, 0, s, a); \
    return hipGetLastError();                                                                    \
  }
#define LSQ_PF_PG(B, DK, DV) \
  LSQ_PF(B, DK, DV, dev::POL_DYNAMIC, 0) LSQ_PF(B, DK, DV, dev::POL_DYNAMIC, 1) \
  LSQ_PF(B, DK, DV, dev::POL_PERSISTENT, 0) LSQ_PF(B, DK, DV, dev::POL_PERSISTENT, 1)
  LSQ_PF_PG(4, 128, 128) LSQ_PF_PG(4, 128, 64) LSQ_PF_PG(4, 64, 128) LSQ_PF_PG(4, 64, 64)
  LSQ_PF_PG(8, 128, 128) LSQ_PF_PG(8, 128, 64) LSQ_PF_PG(8, 64, 128) LSQ_PF_PG(8, 64, 64)
#undef LSQ_PF_PG
#undef LSQ_PF
  return hipErrorInvalidValue;
}

}  // namespace lsq
