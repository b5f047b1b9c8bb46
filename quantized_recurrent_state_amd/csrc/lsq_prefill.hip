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
  constexpr int TR = DV / 64;            // tile rows per wave
  constexpr int TC = DK / 16;            // tile columns
  constexpr int ROWB = DK * BITS / 8;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int h = blockIdx.x;
  const int ng = a.ng, g = a.group;

  __shared__ __align__(16) int8_t vt[DV * kOpRow];      // (B V)^T codes [dv][token]
  __shared__ __align__(16) int8_t kt[DK * kOpRow];      // (Gamma-> K)^T codes [dk][token]
  __shared__ __align__(16) int8_t stage[DV * DK];       // state codes [dv][dk]
  __shared__ float sscale[DV * 8];                      // state scales [dv][ng] (ng <= 8)
  __shared__ float gam[DK];                             // gamma^C per column
  __shared__ unsigned amax_bits[2];                     // operand block maxima (V, K)

  const size_t hrow0 = (size_t)h * DV;
  // ---- the head's packed state -> LDS codes and scales
  for (int idx = tid; idx < DV * DK; idx += 256) {
    const int r = idx / DK, c = idx % DK;
    const uint8_t byte = a.codes[(hrow0 + r) * ROWB + (BITS == 4 ? c / 2 : c)];
    int code;
    if constexpr (BITS == 4) code = ((int)(((c & 1) ? (byte >> 4) : byte) & 0xF) ^ 8) - 8;
    else code = (int)(int8_t)byte;
    stage[idx] = (int8_t)code;
  }
  for (int idx = tid; idx < DV * ng; idx += 256) sscale[idx] = a.scales[hrow0 * ng + idx];
  __syncthreads();
  // dequantised state in the accumulator layout: S[I][J][v]
  float S[TR][TC][4];
#pragma unroll
  for (int I = 0; I < TR; ++I)
#pragma unroll
    for (int J = 0; J < TC; ++J)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int r = 16 * (wave * TR + I) + 4 * (lane / 16) + v, c = 16 * J + (lane % 16);
        S[I][J][v] = (float)stage[r * DK + c] * sscale[r * ng + c / g];
      }

  const int64_t nh = a.n_heads;
  for (int t0 = 0; t0 < a.T; t0 += kChunk) {
    const int tc = min(kChunk, a.T - t0);
    // ---- operands: one column per thread, the chunk's tokens in registers
    float col[kChunk];
    float cmax = 0.f;
    const bool krole = tid < DK, vrole = tid >= 128 && tid < 128 + DV;
    if (krole) {
      float acc = 1.f;                   // Gamma->: product of the later tokens' decays
#pragma unroll
      for (int t = kChunk - 1; t >= 0; --t) {
        col[t] = 0.f;
        if (t < tc) {
          const int64_t row = (int64_t)(t0 + t) * nh + h;
          col[t] = acc * a.k[row * DK + tid];
          acc = acc * (DIAG ? a.alpha[row * DK + tid] : a.alpha[row]);
        }
        cmax = fmaxf(cmax, fabsf(col[t]));
      }
      gam[tid] = acc;
    } else if (vrole) {
      const int i = tid - 128;
#pragma unroll
      for (int t = 0; t < kChunk; ++t) {
        col[t] = 0.f;
        if (t < tc) {
          const int64_t row = (int64_t)(t0 + t) * nh + h;
          col[t] = a.beta[row] * a.v[row * DV + i];
        }
        cmax = fmaxf(cmax, fabsf(col[t]));
      }
    }
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
    // ---- H = (B V)^T (Gamma-> K) on the matrix cores
    i32x4 acc[TR][TC];
#pragma unroll
    for (int I = 0; I < TR; ++I)
#pragma unroll
      for (int J = 0; J < TC; ++J) acc[I][J] = i32x4{0, 0, 0, 0};
#pragma unroll
    for (int ks = 0; ks < kChunk / 32; ++ks) {
      const int koff = 32 * ks + 8 * (lane / 16);
      long bop[TC];
#pragma unroll
      for (int J = 0; J < TC; ++J)
        bop[J] = *reinterpret_cast<const long*>(&kt[(16 * J + lane % 16) * kOpRow + koff]);
#pragma unroll
      for (int I = 0; I < TR; ++I) {
        const long aop =
            *reinterpret_cast<const long*>(&vt[(16 * (wave * TR + I) + lane % 16) * kOpRow + koff]);
#pragma unroll
        for (int J = 0; J < TC; ++J)
          acc[I][J] = __builtin_amdgcn_mfma_i32_16x16x32_i8(aop, bop[J], acc[I][J], 0, 0, 0);
      }
    }
    // ---- state pass: X = fma(gamma, S, H), requantised per group
    const float sc = s_v * s_k;
    const bool last = t0 + kChunk >= a.T;
#pragma unroll
    for (int I = 0; I < TR; ++I)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int r = 16 * (wave * TR + I) + 4 * (lane / 16) + v;
        float x[TC];
#pragma unroll
        for (int J = 0; J < TC; ++J) {
          const int c = 16 * J + lane % 16;
          const float H = (float)acc[I][J][v] * sc;
          x[J] = fmaf(gam[DIAG ? c : 0], S[I][J][v], H);
        }
        // groups of g columns: g/16 tiles (an aligned power of two) x the 16
        // lanes of a DPP row; butterflies over tiles keep every index static
        const int tpg = g / 16;
        float s[TC];
        if constexpr (POLICY == POL_DYNAMIC) {
          float m[TC];
#pragma unroll
          for (int J = 0; J < TC; ++J) m[J] = fabsf(x[J]);
#pragma unroll
          for (int step = 1; step < TC; step *= 2) {
            if (step < tpg) {
              float n2[TC];
#pragma unroll
              for (int J = 0; J < TC; ++J) n2[J] = fmaxf(m[J], m[J ^ step]);
#pragma unroll
              for (int J = 0; J < TC; ++J) m[J] = n2[J];
            }
          }
#pragma unroll
          for (int J = 0; J < TC; ++J) {
            s[J] = group_max(m[J], 16) / QMAX;
            if (lane % 16 == 0 && (J % tpg) == 0) sscale[r * ng + (16 * J) / g] = s[J];
          }
        } else {
#pragma unroll
          for (int J = 0; J < TC; ++J) s[J] = sscale[r * ng + (16 * J) / g];
        }
#pragma unroll
        for (int J = 0; J < TC; ++J) {
          const int code = rne_code(x[J], inv_scale(s[J]), QMAX);
          S[I][J][v] = (float)code * s[J];
          if (last) stage[r * DK + 16 * J + lane % 16] = (int8_t)code;
        }
      }
    __syncthreads();
  }
  if (a.T <= 0) return;
  // ---- LDS codes and scales -> the head's packed state
  for (int idx = tid; idx < DV * ROWB; idx += 256) {
    const int r = idx / ROWB, b = idx % ROWB;
    uint8_t byte;
    if constexpr (BITS == 4)
      byte = (uint8_t)((stage[r * DK + 2 * b] & 0xF) | ((stage[r * DK + 2 * b + 1] & 0xF) << 4));
    else
      byte = (uint8_t)stage[r * DK + b];
    a.codes[(hrow0 + r) * ROWB + b] = byte;
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
