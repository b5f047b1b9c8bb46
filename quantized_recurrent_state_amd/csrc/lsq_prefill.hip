// Chunkwise prefill state pass (linear write, delta = 0) on the matrix cores.
//
// "LinQuant: Functional Invariances for Low-Precision Linear Recurrences"
// (summary page), Methodology, Low-Precision Chunkwise Realization: per chunk
// of C tokens the state write H = Q(B V)^T Q(Gamma-> (.) K) and the state pass
// S_[i+1] = Q(gamma^C S_[i] + H).  Reading (the oracle's): Gamma->_t is the
// fp32 suffix product of the chunk's later decays, gamma^C the chunk's
// product; B V = fl(beta v); one INT8 absmax scale per operand block (head,
// chunk); the integer product is exact, H = fl(h fl(s_V s_K)); X = fma(gamma,
// S, H) requantised in the state's group format and policy (RNE); S carried as
// fl(code s).
//
// One workgroup (four waves) per head walks the chunks in order.  Per chunk:
//   operands   thread c < Dk builds column c of Gamma-> (.) K (its decay
//              suffix product in the oracle's order), thread 128 + i column i
//              of B V, 64 tokens each in registers; block absmax (LDS max);
//              INT8 codes written transposed ([column][token], rows padded to
//              72 bytes) to LDS;
//   H          v_mfma_i32_16x16x32_i8: A = (B V)^T tile rows, B = K tile
//              columns, two k-steps of 32 tokens; wave w owns tile rows
//              w*R .. w*R+R-1 (R = Dv/64) and every tile column;
//   state pass in the accumulator layout (lane l: column 16J + l%16, rows
//              16I + 4(l/16) + v): the group absmax is a DPP reduction over
//              the 16 lanes of a DPP row and the group's tiles.
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

template <int BITS, int DK, int DV, int POLICY, int DIAG>
__global__ __launch_bounds__(256) void prefill_kernel(PrefillArgs a) {
  constexpr float QMAX = BITS == 4 ? 7.f : 127.f;
  constexpr int RT = DV / 64;            // 16-row tiles per wave
  constexpr int CT = DK / 16;            // 16-column tiles
  constexpr int ROWB = DK * BITS / 8;    // packed bytes per state row
  constexpr int SP = DK + 8;             // LDS pitch of a state code row (bank spread)
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int h = blockIdx.x;
  const int ng = a.ng, g = a.group;

  __shared__ __align__(16) int8_t vt[DV * kOpRow];      // (B V)^T codes [dv][token]
  __shared__ __align__(16) int8_t kt[DK * kOpRow];      // (Gamma-> K)^T codes [dk][token]
  __shared__ __align__(16) int8_t stage[DV * SP];       // state codes [dv][dk]
  __shared__ float sscale[DV * 8];                      // state scales [dv][ng] (ng <= 8)
  __shared__ __align__(16) float gam[DK];               // gamma^C per column
  __shared__ unsigned amax_bits[2];                     // operand block maxima (V, K)

  // ---- the head's packed state -> LDS codes and scales.  The state stays
  // there as codes between chunks: the carried value is fl(code * scale).
  const size_t hrow0 = (size_t)h * DV;
  const uint32_t* gcodes = reinterpret_cast<const uint32_t*>(a.codes + hrow0 * ROWB);
  for (int idx = tid; idx < DV * ROWB / 4; idx += 256) {
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
  for (int idx = tid; idx < DV * ng; idx += 256) sscale[idx] = a.scales[hrow0 * ng + idx];
  __syncthreads();

  const int64_t nh = a.n_heads;
  // Operand roles (wave-uniform): waves covering threads c < Dk own column c
  // of Gamma-> (.) K, waves covering threads 128 + i own column i of B V.  A
  // thread's raw inputs for one chunk are p0[t] (k or v) and p1[t] (its decay,
  // or beta), loaded one chunk ahead so that the next chunk's reads are in
  // flight during this chunk's product and state pass.
  const bool krole = wave * 64 < DK, vrole = wave >= 2 && (wave - 2) * 64 < DV;
  const unsigned ut = threadIdx.x;       // unsigned lane offset: scalar base + vector offset loads
  float p0[kChunk], p1[kChunk];
  auto load_chunk = [&](int c0) {
    const int last_t = min(kChunk, a.T - c0) - 1;   // a short chunk re-reads its last token
    if (krole) {
#pragma unroll
      for (int t = 0; t < kChunk; ++t) {
        const int64_t row = (int64_t)(c0 + min(t, last_t)) * nh + h;
        const float* kr = a.k + row * DK;           // uniform row base, lane offset
        p0[t] = kr[ut];
        if constexpr (DIAG) {
          const float* ar = a.alpha + row * DK;
          p1[t] = ar[ut];
        } else {
          p1[t] = a.alpha[row];
        }
      }
    } else if (vrole) {
#pragma unroll
      for (int t = 0; t < kChunk; ++t) {
        const int64_t row = (int64_t)(c0 + min(t, last_t)) * nh + h;
        const float* vr = a.v + row * DV;
        p0[t] = vr[ut - 128u];
        p1[t] = a.beta[row];
      }
    }
  };
  if (a.T > 0) load_chunk(0);

  for (int t0 = 0; t0 < a.T; t0 += kChunk) {
    const int tc = min(kChunk, a.T - t0);
    // ---- operands: one column per thread, the chunk's tokens in registers
    float col[kChunk];
    float cmax = 0.f;
    if (krole) {
      float acc = 1.f;                   // Gamma->: product of the later tokens' decays
#pragma unroll
      for (int t = kChunk - 1; t >= 0; --t) {
        const bool in = t < tc;
        col[t] = in ? acc * p0[t] : 0.f;
        acc = in ? acc * p1[t] : acc;
        cmax = fmaxf(cmax, fabsf(col[t]));
      }
      gam[tid] = acc;
    } else if (vrole) {
#pragma unroll
      for (int t = 0; t < kChunk; ++t) {
        col[t] = t < tc ? p1[t] * p0[t] : 0.f;
        cmax = fmaxf(cmax, fabsf(col[t]));
      }
    }
    if (t0 + kChunk < a.T) load_chunk(t0 + kChunk);
    if (tid < 2) amax_bits[tid] = 0u;
    __syncthreads();
    if (krole) atomicMax(&amax_bits[1], __float_as_uint(cmax));
    if (vrole) atomicMax(&amax_bits[0], __float_as_uint(cmax));
    __syncthreads();
    const float s_v = __uint_as_float(amax_bits[0]) / 127.f;
    const float s_k = __uint_as_float(amax_bits[1]) / 127.f;
    if (krole || vrole) {
      const float inv = inv_scale(krole ? s_k : s_v);
      int8_t* dst = krole ? &kt[tid * kOpRow] : &vt[(tid - 128) * kOpRow];
#pragma unroll
      for (int t4 = 0; t4 < kChunk / 4; ++t4) {
        uint32_t w = 0;
#pragma unroll
        for (int q = 0; q < 4; ++q) w |= (uint32_t)(rne_code(col[4 * t4 + q], inv, 127.f) & 0xFF) << (8 * q);
        reinterpret_cast<uint32_t*>(dst)[t4] = w;
      }
    }
    __syncthreads();
    // ---- H on the matrix cores: A = (Gamma-> K) codes (rows = state columns),
    // B = (B V) codes (columns = state rows), so that lane l receives
    // H[16(wave RT + J) + l%16][16 I + 4(l/16) + v], v = 0..3: four adjacent
    // columns of one state row per tile
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
        bv[J] = *reinterpret_cast<const long*>(&vt[(16 * (wave * RT + J) + lane % 16) * kOpRow + koff]);
#pragma unroll
      for (int I = 0; I < CT; ++I) {
        const long ak = *reinterpret_cast<const long*>(&kt[(16 * I + lane % 16) * kOpRow + koff]);
#pragma unroll
        for (int J = 0; J < RT; ++J)
          acc[J][I] = __builtin_amdgcn_mfma_i32_16x16x32_i8(ak, bv[J], acc[J][I], 0, 0, 0);
      }
    }
    // ---- state pass: X = fma(gamma, S, H), requantised per group
    const float sc = s_v * s_k;
    const int tpg = g / 16;              // tiles per group (an aligned power of two)
    float gc[CT][4];
#pragma unroll
    for (int I = 0; I < CT; ++I) {
      if constexpr (DIAG) {
        const float4 q4 = *reinterpret_cast<const float4*>(&gam[16 * I + 4 * (lane / 16)]);
        gc[I][0] = q4.x; gc[I][1] = q4.y; gc[I][2] = q4.z; gc[I][3] = q4.w;
      } else {
#pragma unroll
        for (int v = 0; v < 4; ++v) gc[I][v] = gam[0];
      }
    }
#pragma unroll
    for (int J = 0; J < RT; ++J) {
      const int r = 16 * (wave * RT + J) + lane % 16;
      int8_t* crow = &stage[r * SP + 4 * (lane / 16)];
      float x[CT][4], s[CT];
#pragma unroll
      for (int I = 0; I < CT; ++I) {
        const uint32_t cw = *reinterpret_cast<const uint32_t*>(&crow[16 * I]);
        s[I] = sscale[r * ng + (16 * I) / g];
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const float S = (float)(int)(int8_t)(cw >> (8 * v)) * s[I];
          x[I][v] = fmaf(gc[I][v], S, (float)acc[J][I][v] * sc);
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
  if (a.T <= 0) return;
  // ---- LDS codes and scales -> the head's packed state
  uint32_t* ocodes = reinterpret_cast<uint32_t*>(a.codes + hrow0 * ROWB);
  for (int idx = tid; idx < DV * ROWB / 4; idx += 256) {
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
  if constexpr (POLICY == POL_DYNAMIC) {
    for (int idx = tid; idx < DV * ng; idx += 256) a.scales[hrow0 * ng + idx] = sscale[idx];
  }
}

}  // namespace dev

hipError_t launch_prefill(const PrefillArgs& a, int bits, int dk, int dv, int policy, int diag,
                          hipStream_t s) {
  const dim3 grid(a.n_heads), block(256);
#define LSQ_PF(B, DK, DV, P, G)                                                                   \
  if (bits == B && dk == DK && dv == DV && policy == P && diag == G) {                           \
    hipLaunchKernelGGL((dev::prefill_kernel<B, DK, DV, P, G>), grid, block, 0, s, a);            \
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
