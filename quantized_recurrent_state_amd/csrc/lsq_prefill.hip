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

// max of x over the four lanes l, l^16, l^32, l^48 (the lanes that hold one
// state row): the gfx950 row-swap instructions, no LDS round trip.
__device__ __forceinline__ float max_across_rows(float x) {
  const uint32_t u = __float_as_uint(x);
  const auto p = __builtin_amdgcn_permlane16_swap(u, u, false, false);
  x = fmaxf(__uint_as_float(p[0]), __uint_as_float(p[1]));
  const uint32_t w = __float_as_uint(x);
  const auto q = __builtin_amdgcn_permlane32_swap(w, w, false, false);
  return fmaxf(__uint_as_float(q[0]), __uint_as_float(q[1]));
}

// fl(m / qmax) for qmax = 7 (INT4) or 127 (INT8): the product with fl(1/qmax),
// its exact residual and one corrective fma.  Equal to the IEEE quotient for
// every finite m >= 0 (checked over all finite floats for both divisors);
// m = +inf gives NaN, which the caller's range check sends to IEEE division.
template <int BITS>
__device__ __forceinline__ float div_qmax(float m) {
  constexpr float QM = BITS == 4 ? 7.f : 127.f;
  constexpr float C = 1.f / QM;
  const float q = m * C;
  const float r = fmaf(-q, QM, m);
  return fmaf(r, C, q);
}

// fl(1/s) for s in [2^-126, 2^126): v_rcp_f32 and one Newton step (the
// decode step's reciprocal without its out-of-range branch).
__device__ __forceinline__ float rcp_newton(float s) {
  const float r0 = __builtin_amdgcn_rcpf(s);
  const float e = fmaf(-s, r0, 1.0f);
  return fmaf(e, r0, r0);
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
  constexpr int OPC = 128 + DV;                          // staged operand columns: K at c, V at 128 + row
  __shared__ float colbuf[kChunk * OPC];                // fp32 operand columns of the next chunk [token][column]
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

  // One operand role (K side or V side), as a loop of its own: nchunk + 2
  // iterations with one barrier each.  The reads of the next chunk to build
  // are issued one iteration before they are used, so that their HBM latency
  // overlaps a whole iteration; every read is unconditional within the loop
  // (no register copy of a read value, which would wait for all reads in
  // flight).
  auto operand_loop = [&](auto kside) {
    constexpr bool K = decltype(kside)::value;
    constexpr bool TOK = !(K && DIAG);   // a per-token scalar (scalar decay, beta): lane t, token t
    const int col_c = K ? tid : tid - 128;
    float v0[kChunk], v1[TOK ? 1 : kChunk];
    float pl = 0.f;
    float gh = 1.f;                      // gamma^C of the chunk last built (K side)
    // reads of chunk p (p < nchunk); a short chunk re-reads its last token
    auto read_chunk = [&](int p) {
      const int c0 = p * kChunk;
      const int tm = min(kChunk, a.T - c0) - 1;
      const int64_t row0 = (int64_t)c0 * nh + h;
      const int64_t s0 = nh * (K ? DK : DV);
      const float* r = K ? a.k + row0 * DK : a.v + row0 * DV - 128;
#pragma unroll
      for (int t = 0; t < kChunk; ++t) {
        v0[t] = r[ut];
        if (t < tm) r += s0;
      }
      if constexpr (!TOK) {
        const float* ra = a.alpha + row0 * DK;
#pragma unroll
        for (int t = 0; t < kChunk; ++t) {
          v1[t] = ra[ut];
          if (t < tm) ra += s0;
        }
      } else {
        pl = (K ? a.alpha : a.beta)[row0 + (int64_t)min(lane, tm) * nh];
      }
    };
    float* mycol = &colbuf[tid];         // this thread's operand column, token stride OPC
    if (nchunk > 0) read_chunk(0);
    for (int i = -2; i < nchunk; ++i) {
      // ---- (a) quantise chunk i+1's columns with the posted block maxima
      const int q = i + 1;
      if (q >= 0 && q < nchunk) {
        const int slot = q & 1;
        float m = wmax[slot][K ? 0 : 2];
        if ((K ? KW : VW) > 1) m = fmaxf(m, wmax[slot][K ? 1 : 3]);
        const float sq = m / 127.f;
        const float inv = inv_scale(sq);
        int8_t* dst = K ? &kt[slot][col_c * kOpRow] : &vt[slot][col_c * kOpRow];
#pragma unroll
        for (int t4 = 0; t4 < kChunk / 4; ++t4) {
          uint32_t w = 0;
#pragma unroll
          for (int b = 0; b < 4; ++b)
            w |= (uint32_t)(rne_code(mycol[(4 * t4 + b) * OPC], inv, 127.f) & 0xFF) << (8 * b);
          reinterpret_cast<uint32_t*>(dst)[t4] = w;
        }
        if constexpr (K) gam[slot][col_c] = gh;
        if (col_c == 0) opscale[slot][K ? 1 : 0] = sq;
      }
      // ---- (b) build chunk i+2's operand columns from its reads (into LDS,
      // over the values (a) has just taken), then read chunk i+3 (the last
      // chunk again when there is none: its lines are still in the cache)
      const int p = i + 2;
      if (p < nchunk) {
        const int tc = min(kChunk, a.T - p * kChunk);
        float cmax = 0.f;
        if constexpr (K) {
          float acc = 1.f;               // Gamma->: product of the later tokens' decays
#pragma unroll
          for (int t = kChunk - 1; t >= 0; --t) {
            const bool in = t < tc;
            const float dec =
                TOK ? __int_as_float(__builtin_amdgcn_readlane(__float_as_int(pl), t)) : v1[TOK ? 0 : t];
            const float c = in ? acc * v0[t] : 0.f;
            acc = in ? acc * dec : acc;
            mycol[t * OPC] = c;
            cmax = fmaxf(cmax, fabsf(c));
          }
          gh = acc;
        } else {
#pragma unroll
          for (int t = 0; t < kChunk; ++t) {
            const float b = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(pl), t));
            const float c = t < tc ? b * v0[t] : 0.f;
            mycol[t * OPC] = c;
            cmax = fmaxf(cmax, fabsf(c));
          }
        }
        cmax = wave_max(cmax);
        if (lane == 0) wmax[p & 1][wave] = cmax;
        // the next reads stay below this chunk's last use of v0, v1 and pl,
        // so that they land in the same registers
        asm volatile("" ::: "memory");
        read_chunk(min(p + 1, nchunk - 1));
      }
      if constexpr (XB) __syncthreads();   // the state waves' head maximum
      __syncthreads();
    }
  };

  if (krole) {
    operand_loop(std::true_type{});
  } else if (vrole) {
    operand_loop(std::false_type{});
  } else if (!swave) {                   // no operand role at this shape: the barriers only
    for (int i = -2; i < nchunk; ++i) {
      if constexpr (XB) __syncthreads();
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
        float m[CT];                     // group maxima (dynamic)
        if constexpr (POLICY == POL_DYNAMIC) {
          // group absmax: the tile's four columns in the lane, the group's
          // tiles by butterflies (static indices), then the four lanes that
          // hold the row (l%16 fixed)
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
          for (int I = 0; I < CT; ++I) m[I] = max_across_rows(m[I]);
#pragma unroll
          for (int I = 0; I < CT; ++I) {
            s[I] = div_qmax<BITS>(m[I]);
            // a 16-bit format: the stored value forms the codes
            if constexpr (S16) s[I] = scale_from16(scale_to16(s[I], a.sfmt), a.sfmt);
          }
        }
        // reciprocals of every tile's scale; lanes holding a zero, tiny, huge
        // or non-finite scale (or group maximum) redo theirs with IEEE
        // division, in one branch for all the tiles
        float inv[CT];
        bool slow = false;
#pragma unroll
        for (int I = 0; I < CT; ++I) {
          inv[I] = rcp_newton(s[I]);
          slow = slow || !(s[I] >= 0x1p-126f && s[I] < 0x1p126f);
        }
        if (__builtin_expect(slow, 0)) {
#pragma unroll
          for (int I = 0; I < CT; ++I) {
            if constexpr (POLICY == POL_DYNAMIC) {
              s[I] = m[I] / QMAX;
              if constexpr (S16) s[I] = scale_from16(scale_to16(s[I], a.sfmt), a.sfmt);
            }
            inv[I] = inv_scale(s[I]);
          }
        }
        if constexpr (POLICY == POL_DYNAMIC) {
          if (lane < 16) {
#pragma unroll
            for (int I = 0; I < CT; ++I)
              if ((I % tpg) == 0) sscale[r * ng + (16 * I) / g] = s[I];
          }
        }
#pragma unroll
        for (int I = 0; I < CT; ++I) {
          uint32_t nw = 0;
#pragma unroll
          for (int v = 0; v < 4; ++v) nw |= (uint32_t)(rne_code(x[I][v], inv[I], QMAX) & 0xFF) << (8 * v);
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
